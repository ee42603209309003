// Register and LDS helpers shared by the TTT-Linear matrix-core kernels (linear.hip,
// linear_chunk.hip): bf16 packing and hi/lo splits, lane sums over a DPP row, and reads of a
// token-major tile of 64-wide bf16 rows (128 bytes) whose row r keeps 16-byte chunk c at chunk
// c ^ (r % 8).
#pragma once
#include "common.hpp"

namespace ttt {
namespace {

constexpr int DH = 64;

__device__ __forceinline__ uint2 pack4bf(const float (&v)[4]) {
  return make_uint2(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]));
}

// hi/lo bf16 pairs of four fp32 values: hi = bf16(v), lo = bf16(v - hi), both round to nearest
// even, two values per packed conversion (the hi parts' exact fp32 values are their bits
// shifted into place).
__device__ __forceinline__ void split4(const float (&v)[4], uint2& hi, uint2& lo) {
  const uint32_t h01 = pack2bf(v[0], v[1]), h23 = pack2bf(v[2], v[3]);
  const float r0 = v[0] - __uint_as_float(h01 << 16);
  const float r1 = v[1] - __uint_as_float(h01 & 0xFFFF0000u);
  const float r2 = v[2] - __uint_as_float(h23 << 16);
  const float r3 = v[3] - __uint_as_float(h23 & 0xFFFF0000u);
  hi = make_uint2(h01, h23);
  lo = make_uint2(pack2bf(r0, r1), pack2bf(r2, r3));
}

__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }

// Sum over the 16 lanes of a DPP row (lanes 16k .. 16k+15), result in every lane of the row:
// swaps within quads, then the half-row and row mirrors pair the quads and the halves.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

// 8 bytes at logical element e (a multiple of 4) of token row r
__device__ __forceinline__ uint2 t_rd8(const char* tb, int r, int e) {
  return *reinterpret_cast<const uint2*>(tb + r * 128 + (((e >> 3) ^ (r & 7)) << 4) + (e & 4) * 2);
}
// 16 bytes at logical element e (a multiple of 8) of token row r
__device__ __forceinline__ uint4 t_rd16(const char* tb, int r, int e) {
  return *reinterpret_cast<const uint4*>(tb + r * 128 + (((e >> 3) ^ (r & 7)) << 4));
}
// Transposing read: lane j of each 16-lane group addresses token row r0 + j / 4, elements
// c0 + 4 (j % 4); lane l then holds elements c0 + l % 16 of token rows r0 .. r0 + 3.
__device__ __forceinline__ uint2 t_tr(const char* tb, int r0, int c0, int cl) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int r = r0 + (cl >> 2), e = c0 + 4 * (cl & 3);
  const char* p = tb + r * 128 + (((e >> 3) ^ (r & 7)) << 4) + (e & 4) * 2;
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

}  // namespace
}  // namespace ttt
