// ssm_mfma.h -- bf16 matrix-core helpers shared by the masked-matrix (SSD)
// kernels: operand packing, the bf16 high/low split of fp32 values, the
// gfx950 16x16x32 bf16 MFMA and identity-product transposes.
//
// MFMA lane layout (v_mfma_f32_16x16x32_bf16; 16 x 16 tiles, lane l,
// g = l / 16):
//   A operand: row l % 16, contraction slots 8g..8g+7
//   B operand: column l % 16, the same slots
//   result:    column l % 16, rows 4g..4g+3
#pragma once

#include "ssm_device.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_bf16(float lo_elem, float hi_elem) {
  bf16x2_t v = {(__bf16)lo_elem, (__bf16)hi_elem};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// (a, b) ~= hi + lo with hi, lo packed bf16 pairs: hi = rounded value, lo =
// rounded remainder (the remainder itself is exact in fp32).  The high part
// of a is moved into place with a byte permute (v_perm_b32: bytes 1:0 of hi
// to 3:2, zeros below), which the compiler keeps as one instruction.
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  const float ah = __uint_as_float(__builtin_amdgcn_perm(0u, hi, 0x01000c0cu));
  lo = pack_bf16(a - ah, b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ f32x4_t mfma_k32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t lds128(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ u32x2_t lds64(const uint16_t* p) {
  return *reinterpret_cast<const u32x2_t*>(p);
}
__device__ __forceinline__ u32x4_t cat(u32x2_t a, u32x2_t b) { return {a.x, a.y, b.x, b.y}; }

// Four values that are bf16 numbers (results of an identity product) as two
// packed words; the conversion is exact.
__device__ __forceinline__ u32x2_t to_bf16x4(f32x4_t v) {
  return {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}

// B operand of an identity product that picks 16 of the A operand's 32
// contraction columns: lane (column c = l % 16, slots k = 8g..8g+7) holds 1
// where k == off + c.  A x I_off is then the 16 x 16 tile A[:, off..off+15] in
// the result layout (column c, rows 4g..4g+3), which is the operand layout of
// a product contracting over those rows: the transposes the contractions need
// are done on the matrix cores instead of through LDS.
__device__ __forceinline__ u32x4_t identity_pick(int off, int r16, int g) {
  uint32_t wv[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t lo = (8 * g + 2 * m == off + r16) ? 0x3f80u : 0u;      // bf16 1.0
    const uint32_t hi = (8 * g + 2 * m + 1 == off + r16) ? 0x3f80u : 0u;
    wv[m] = lo | (hi << 16);
  }
  return {wv[0], wv[1], wv[2], wv[3]};
}

// B operand of the identity for an A operand that fills slots 0..3 of each
// lane group with contraction index 4g + s (slots 4..7 zero): lane (column c,
// group g) holds 1 in slot s < 4 where 4g + s == c.
__device__ __forceinline__ u32x4_t identity_pick4(int r16, int g) {
  const uint32_t e0 = (4 * g == r16) ? 0x3f80u : 0u, e1 = (4 * g + 1 == r16) ? 0x3f80u : 0u;
  const uint32_t e2 = (4 * g + 2 == r16) ? 0x3f80u : 0u, e3 = (4 * g + 3 == r16) ? 0x3f80u : 0u;
  return {e0 | (e1 << 16), e2 | (e3 << 16), 0u, 0u};
}

}  // namespace
}  // namespace ssm
