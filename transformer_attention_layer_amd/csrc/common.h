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

GQA_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
GQA_DEV u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
GQA_DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
GQA_DEV void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

GQA_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

GQA_DEV float bf16_to_f32(bf16 v) { return (float)v; }

// Round-to-nearest-even float -> bf16 bits (two values packed, low first).
GQA_DEV unsigned int pack_bf16x2(float lo, float hi) {
  bf16 a = (bf16)lo;
  bf16 b = (bf16)hi;
  return (unsigned int)__builtin_bit_cast(unsigned short, a) |
         ((unsigned int)__builtin_bit_cast(unsigned short, b) << 16);
}

GQA_DEV float lo_bf16(unsigned int w) { return __builtin_bit_cast(float, w << 16); }
GQA_DEV float hi_bf16(unsigned int w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// D = A(32x16) * B(16x32) + C on the bf16 matrix cores (gfx950).  Lane l
// supplies row l%32 of A and column l%32 of B, eight K-values each; lane l,
// register r of D is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
GQA_DEV floatx16 mfma32x32x16(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

GQA_DEV float wave_xor32(float v) { return __shfl_xor(v, 32, 64); }

GQA_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
