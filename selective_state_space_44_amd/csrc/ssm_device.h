// ssm_device.h -- small device helpers shared by the scan and decode kernels
// (gfx950, wave64).  Internal header; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr int kWave = 64;
constexpr int kDState = 16;
// log2(e): exp(v) is evaluated as exp2(v * log2(e)) on the hardware exp2.
constexpr float kLog2e = 1.4426950408889634f;

// bf16 is carried as its 16 raw bits.
struct bf16 { uint16_t bits; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename IO> struct io;
template <> struct io<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct io<bf16> {
  __device__ __forceinline__ static float load(const bf16* p) {
    return bf16_bits_to_f32(p->bits);
  }
  __device__ __forceinline__ static void store(bf16* p, float v) {
    p->bits = f32_to_bf16_bits(v);
  }
};

// Hardware exp2 (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// SiLU(v) = v * sigmoid(v) = v / (1 + exp(-v)).
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
}

// Raw buffer resource over [base, base + bytes) for loads/stores addressed
// by a per-lane byte offset (VGPR) plus a wave-uniform byte offset (SGPR), so
// that stepping through rows costs scalar adds only.  Accesses at or beyond
// `bytes` (relative to base, lane offset) read 0 / are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // 0x00020000: dword 3 of a raw (untyped, stride 0) buffer descriptor on gfx9.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <typename IO> struct buf;
template <> struct buf<float> {
  __device__ __forceinline__ static float load(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
  }
  __device__ __forceinline__ static void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
  }
};
template <> struct buf<bf16> {
  __device__ __forceinline__ static float load(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
    return bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
  }
  __device__ __forceinline__ static void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(v), r, voff, soff, 0);
  }
};

// Wave index inside the block as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

}  // namespace ssm
