// Device-side helpers shared by the gfx950 kernels: bf16 packing, CDNA4 matrix-core wrappers
// and the launch-side declarations each kernel file implements.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> fp32 value (exact).
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> one dword holding two bf16 (low half = a), round to nearest even: one packed
// conversion instruction on gfx950.
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Element load as fp32 for the two input dtypes.
__device__ __forceinline__ float ld_elem(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld_elem(const uint16_t* p, size_t i) { return bf2f(p[i]); }

__device__ __forceinline__ void st_elem(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_elem(uint16_t* p, size_t i, float v) { p[i] = f2bf(v); }

// D += A * B on a 32x32 output block, K = 16, bf16 operands (gfx950 v_mfma_f32_32x32x16_bf16).
// Operand lane layout: lane l supplies row (l % 32) of A / column (l % 32) of B, with the eight
// K values 8*(l/32) .. 8*(l/32)+7. Result: lane l holds column l % 32, rows
// 8*(j/4) + 4*(l/32) + (j%4) for j = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const uint4& a, const uint4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D += A * B on a 16x16 block, K = 32 (gfx950 v_mfma_f32_16x16x32_bf16): lane l supplies row /
// column l % 16 with K values 8*(l/16) .. +7; result lane l holds column l % 16, rows 4*(l/16)+i.
__device__ __forceinline__ f32x4 mfma16x16x32(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D += A * B on a 16x16 block, K = 16 (v_mfma_f32_16x16x16_bf16): lane l supplies row / column
// l % 16 with K values 4*(l/16) .. +3; result layout as for the K = 32 form.
__device__ __forceinline__ f32x4 mfma16x16x16(const uint2& a, const uint2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                   __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
}

// Split v into hi + lo with hi = bf16(v), lo = bf16(v - hi): a two-term bf16 representation
// good to ~16 mantissa bits, used where an fp32 state enters a bf16 product.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}

}  // namespace ttt
