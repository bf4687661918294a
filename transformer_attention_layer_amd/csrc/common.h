// Device-side helpers shared by the gfx950 kernels of the GQA layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define GQA_DEV static __device__ __forceinline__

// 0.5 * log2(e) etc. are formed on the host; log2(e) here for exp2-based softmax.
#define GQA_LOG2E 1.4426950408889634f

// (cos, sin) of position pos at rotary frequency i of `half` (the rotary
// width is 2 half): angle pos * theta^(-2 i / (2 half)), in double, rounded
// to float once.  One definition for the RoPE table and for the kernels that
// evaluate it in place, so both give the same values.
GQA_DEV float2 rope_cos_sin(long pos, int i, int half, double theta) {
  const double inv = pow(theta, -2.0 * (double)i / (double)(2 * half));
  const double ang = (double)pos * inv;
  double sn, cs;
  sincos(ang, &sn, &cs);
  return make_float2((float)cs, (float)sn);
}

GQA_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
GQA_DEV u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
GQA_DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
GQA_DEV void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

GQA_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

GQA_DEV float bf16_to_f32(bf16 v) { return (float)v; }

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float -> bf16 bits (two values packed, low first);
// one v_cvt_pk_bf16_f32.
GQA_DEV unsigned int pack_bf16x2(float lo, float hi) {
  const floatx2 f = {lo, hi};
  const bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(unsigned int, b);
}

// lo + hi of a packed bf16 pair, accumulated into `acc` in fp32 (v_dot2 with
// ones).
GQA_DEV float sum_bf16x2(unsigned int packed, float acc) {
  const bf16x2 v = __builtin_bit_cast(bf16x2, packed);
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(v, ones, acc, false);
}

// Wave-uniform copy of a value (lets the compiler keep it in an SGPR and
// branch on it with scalar branches).
GQA_DEV int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Raw buffer descriptor over `bytes` bytes from `base`; loads at or past the
// end return zero (hardware bounds check).
GQA_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

GQA_DEV void dma16(__amdgpu_buffer_rsrc_t r, void* lds_base, unsigned voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base,
                                           16, voff, 0, 0, 0);
}

GQA_DEV u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, unsigned voff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  u32x4 out;
  out.x = v[0];
  out.y = v[1];
  out.z = v[2];
  out.w = v[3];
  return out;
}

GQA_DEV u32x2 buf_ld8(__amdgpu_buffer_rsrc_t r, unsigned voff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
  u32x2 out;
  out.x = v[0];
  out.y = v[1];
  return out;
}

GQA_DEV float lo_bf16(unsigned int w) { return __builtin_bit_cast(float, w << 16); }
GQA_DEV float hi_bf16(unsigned int w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// D = A(32x16) * B(16x32) + C on the bf16 matrix cores (gfx950).  Lane l
// supplies row l%32 of A and column l%32 of B, eight K-values each; lane l,
// register r of D is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
GQA_DEV floatx16 mfma32x32x16(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// The same product on the fp16 matrix cores: A and B hold fp16 values.
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
GQA_DEV floatx16 mfma32x32x16_f16(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

// D = A(16x32) * B(32x16) + C on the bf16 matrix cores (gfx950).  Lane l
// supplies row l%16 of A and column l%16 of B, eight K-values each (the
// same eight for A and B: K-group l/16); lane l, register r of D is row
// 4*(l/16) + r, column l%16.
GQA_DEV floatx4 mfma16x16x32(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
GQA_DEV floatx4 mfma16x16x32_f16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a),
                                                __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

// Round-to-nearest-even float -> fp16 bits (two values packed, low first);
// one v_cvt_pk_f16_f32.  Magnitudes past 65504 become infinities.
GQA_DEV unsigned int pack_f16x2(float lo, float hi) {
  const floatx2 f = {lo, hi};
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f, halfx2));
}

GQA_DEV float wave_xor32(float v) { return __shfl_xor(v, 32, 64); }

// Combine v across lanes l and l ^ 32 with v_permlane32_swap (a VALU
// instruction, unlike ds_bpermute it does not wait behind this wave's LDS
// reads): swap(v, v) returns v of lanes 0..31 in both halves of its first
// result and v of lanes 32..63 in both halves of its second.
GQA_DEV float max_xor32(float v) {
  const auto q = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)q[0]), __builtin_bit_cast(float, (unsigned)q[1]));
}
// The same over lanes l and l ^ 16 with v_permlane16_swap, which swaps the
// odd 16-lane rows of its first operand with the even rows of its second:
// swap(v, v) returns rows (0, 0, 2, 2) of v and rows (1, 1, 3, 3).
GQA_DEV float sum_xor16(float v) {
  const auto q = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return __builtin_bit_cast(float, (unsigned)q[0]) + __builtin_bit_cast(float, (unsigned)q[1]);
}
GQA_DEV float max_xor16(float v) {
  const auto q = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)q[0]), __builtin_bit_cast(float, (unsigned)q[1]));
}
GQA_DEV float sum_xor32(float v) {
  const auto q = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return __builtin_bit_cast(float, (unsigned)q[0]) + __builtin_bit_cast(float, (unsigned)q[1]);
}

GQA_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Debug builds (libgqa_ldspoison.so, compiled with GQA_LDS_POISON): every
// workgroup first fills its LDS arrays with all-ones bits, a NaN both as
// fp32 and as bf16, and meets at a barrier, so that a read of LDS that
// nothing in the workgroup wrote shows up as a NaN in the results.  The
// release library compiles the calls away.
#ifdef GQA_LDS_POISON
template <typename T, size_t N>
GQA_DEV void poison_one(T (&arr)[N]) {
  unsigned* p = reinterpret_cast<unsigned*>(&arr[0]);
  for (int i = (int)threadIdx.x; i < (int)(sizeof(arr) / 4); i += (int)blockDim.x) p[i] = ~0u;
}
template <typename... A>
GQA_DEV void poison_lds(A&... arrs) {
  (poison_one(arrs), ...);
  __syncthreads();
}
#else
template <typename... A>
GQA_DEV void poison_lds(A&...) {}
#endif
