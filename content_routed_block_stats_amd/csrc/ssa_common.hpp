// Device-side helpers shared by the gfx950 kernels of the SSA hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage type of a bfloat16 tensor element.
struct bf16_t {
  u16 bits;
};

// Storage type of a float16 element (workspace partials).
struct f16_t {
  u16 bits;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bfloat16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ u16 f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(u16, static_cast<__bf16>(f));
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i].bits);
}

template <>
__device__ __forceinline__ float load_f32<f16_t>(const f16_t* p, int64_t i) {
  return static_cast<float>(__builtin_bit_cast(_Float16, p[i].bits));
}

template <typename T>
__device__ __forceinline__ void store_from_f32(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_from_f32<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_from_f32<bf16_t>(bf16_t* p, int64_t i, float v) {
  p[i].bits = f32_to_bf16_bits(v);
}
template <>
__device__ __forceinline__ void store_from_f32<f16_t>(f16_t* p, int64_t i, float v) {
  p[i].bits = __builtin_bit_cast(u16, static_cast<_Float16>(v));
}

// Contraction-index map of one 32x32 MFMA operand fragment.
//
// A 32x32xK MFMA tile gives lane (n = lane%32, h = lane/32) of the result the
// 16 entries (row 8a + 4h + b, column n) for a, b in 0..3.  For a following
// product that contracts over those rows, the same lane must supply exactly
// these 16 values as its operand elements.  Both MFMA operands hand lane
// (., h) the contraction slots of "half h", eight per 16-wide chunk s, so
// pairing operand element e of chunk s in lane half h with the contraction
// index lambda(s, h, e) below makes every lane's operand elements the
// values it already holds:  lambda(2*mt + (a>>1), h, 4*(a&1) + b) = 32*mt + 8a + 4h + b.
__host__ __device__ __forceinline__ constexpr int frag_k(int s, int h, int e) {
  return 16 * s + 8 * (e >> 2) + 4 * h + (e & 3);
}

// One MFMA step contracting a 16-wide chunk: bf16 inputs (one instruction)...
// Two float32 values as a float16 pair (round to nearest even), one
// conversion instruction for both: converting element by element into a
// float16 vector costs a conversion and a merge per value.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}

// Eight float32 values as a float16 MFMA fragment.
__device__ __forceinline__ f16x8 to_f16x8(const float (&v)[8]) {
  return __builtin_bit_cast(f16x8, u32x4{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]),
                                         pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7])});
}

__device__ __forceinline__ floatx16 mma16(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// ...or float16 inputs (one instruction)...
__device__ __forceinline__ floatx16 mma16(const f16x8& a, const f16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// ...or float32 inputs (eight 32x32x2 instructions, element e on slot 2e + h).
__device__ __forceinline__ floatx16 mma16(const floatx8& a, const floatx8& b, floatx16 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace ssa
