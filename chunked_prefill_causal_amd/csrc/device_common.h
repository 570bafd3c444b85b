// Device-side building blocks shared by the gfx950 kernels of libchunkattn.
//
// Matrix-core conventions (CDNA4, wave64), checked on the hardware:
//  * v_mfma_f32_32x32x16_bf16: lane l supplies A[l%32][8*(l/32) + i] and
//    B[8*(l/32) + i][l%32] for i = 0..7; accumulator register r of lane l is
//    D[8*(r/4) + 4*(l/32) + r%4][l%32].
//  * v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and B[l/32][l%32];
//    same accumulator map.
//  * v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8*(l/16) + i] and
//    B[8*(l/16) + i][l%16]; accumulator register r of lane l is
//    D[4*(l/16) + r][l%16].
// Only the pairing of A and B slots matters for a contraction, so each kernel
// is free to choose which key or feature a slot stands for, as long as both
// operands agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace chunkattn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;


// Storage element traits: X elements fill one 16-byte chunk.
template <typename E> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int X = 8; };   // bfloat16 bits
template <> struct Elem<float> { static constexpr int X = 4; };

__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Value of lane l^32 combined with this lane's by `op` (max or add): one
// v_permlane32_swap gives every lane both halves.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats to packed bfloat16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// Online-softmax maximum policy: a row's running maximum is raised only when
// a new logit exceeds it by more than kLazyRescale (log2 units, after the
// scale), so exp2(s - m) stays <= 2^kLazyRescale while O and l are rescaled
// rarely.  Numerator and normaliser share the same offset, so the result is
// exact whatever offset is used.
constexpr float kLazyRescale = 8.0f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ int clamp_block(int32_t id, int32_t num_blocks) {
  return id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
}

// Row merge of split partials stored in log2 units: ml = {m*log2e*scale, l}.
// Partials whose m is -inf (no visible key) carry no weight and their O is
// never read.
__device__ __forceinline__ void merge_weights(const float* ml, int nsplit, int64_t stride,
                                              float& M, float& L) {
  M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s * stride]);
  L = 0.f;
  if (M == -INFINITY) return;
  for (int s = 0; s < nsplit; ++s) {
    const float m = ml[2 * s * stride];
    if (m != -INFINITY) L += ml[2 * s * stride + 1] * fast_exp2(m - M);
  }
}

}  // namespace chunkattn
