// mfma_common.h — matrix-core operand helpers shared by the decode and chunked-prefill kernels
// of libheadq (gfx950). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace headq {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

template <class T, class S>
__device__ __forceinline__ T bitcast(const S& s) {
  static_assert(sizeof(T) == sizeof(S), "size");
  return __builtin_bit_cast(T, s);
}

// Two-bit codes to exact f16 / bf16 operands. A packed word masked with 0x33333333 (or shifted
// right by 2 first) holds one code per nibble; each byte is then one fp4 (e2m1) pair, whose
// values 0, 0.5, 1, 1.5 scaled by 2 are the codes 0..3 exactly (gfx950 packed fp4 conversion,
// low nibble to the low half).
__device__ __forceinline__ uint32_t even_codes(uint32_t w) { return w & 0x33333333u; }
__device__ __forceinline__ uint32_t odd_codes(uint32_t w) { return (w >> 2) & 0x33333333u; }
template <int B>
__device__ __forceinline__ uint32_t fp4_pair_f16(uint32_t m) {
  return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, B));
}
template <int B>
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t m) {
  return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 2.0f, B));
}
// 8 key codes (f16) from a masked word: byte b holds the channel pair (2b, 2b+1) of the run.
__device__ __forceinline__ half8_t key_codes8(uint32_t m) {
  const u32x4 w = {fp4_pair_f16<0>(m), fp4_pair_f16<1>(m), fp4_pair_f16<2>(m), fp4_pair_f16<3>(m)};
  return bitcast<half8_t>(w);
}
// 8 key codes (f16) of a nibble word (3- and 4-bit base codes): the channel pair (2i, 2i+1) is
// nibble i of the low and the high half; or-ing 0x6400 makes each half 1024 + code exactly.
__device__ __forceinline__ half8_t key_codes8_nib(uint32_t w) {
  u32x4 p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
  return bitcast<half8_t>(p) - (half8_t)(_Float16)1024.0f;
}
// 8 value codes (bf16) of one channel tile from a word of the lane's value codes: the low 16 bits
// are tile 2w, the high 16 bits tile 2w+1; even-masked bytes hold token items 0..3, odd-masked
// bytes items 4..7.
template <int HALF>
__device__ __forceinline__ bf16x8_t value_codes8(uint32_t e, uint32_t o) {
  const u32x4 w = {fp4_pair_bf16<2 * HALF>(e), fp4_pair_bf16<2 * HALF + 1>(e), fp4_pair_bf16<2 * HALF>(o),
                   fp4_pair_bf16<2 * HALF + 1>(o)};
  return bitcast<bf16x8_t>(w);
}

// 4 offset-binary nibbles (low 16 bits of x, component i at bits 4i) -> 4 exact f16 values u - 8.
__device__ __forceinline__ half4_t nibbles4_f16(uint32_t x16) {
  const uint32_t y = x16 | (x16 << 12);  // nibble 0 at 0, 1 at 16, 2 at 8, 3 at 24
  u32x2 w;
  w[0] = (y & 0x000F000Fu) | 0x64006400u;  // f16 1024 + u
  w[1] = ((y >> 8) & 0x000F000Fu) | 0x64006400u;
  return bitcast<half4_t>(w) - (half4_t)(_Float16)1032.0f;
}

// x ~ hi + lo with both halves in f16 (hi rounded to nearest, lo the rounded remainder).
__device__ __forceinline__ _Float16 f16_hi(float x) { return (_Float16)x; }
__device__ __forceinline__ _Float16 f16_lo(float x) { return (_Float16)(x - (float)(_Float16)x); }

__device__ __forceinline__ floatx4 mfma_f16(const half8_t& a, const half8_t& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_f16k16(const half4_t& a, const half4_t& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Reductions over the four lanes n, n + 16, n + 32, n + 48 of a wave64 (the four token quads of a
// matrix-product column) in registers: gfx950's lane-row swaps, given one value twice, return at
// every lane its own value and that of the lane 16 (or 32) apart.
__device__ __forceinline__ float partner16_op_max(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float partner32_op_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float quad_max(float x) { return partner32_op_max(partner16_op_max(x)); }
__device__ __forceinline__ float quad_sum(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// x ~ hi + lo in bf16 pairs: hi truncated (the upper half of the f32), lo the remainder rounded
// to nearest; together ~16 significant bits.
__device__ __forceinline__ void split_bf16_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t u0 = bitcast<uint32_t>(x0), u1 = bitcast<uint32_t>(x1);
  hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
  const float2_t r = {x0 - bitcast<float>(u0 & 0xffff0000u), x1 - bitcast<float>(u1 & 0xffff0000u)};
  lo = bitcast<uint32_t>(__builtin_convertvector(r, bf16x2_t));
}

}  // namespace
}  // namespace headq
