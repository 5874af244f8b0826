// ssm_decode.hip -- single-token recurrent decode step for gfx950 (wave64).
//
// One step of the scan's recurrence applied to a resident state
// h[b, d, 0:16] (fp32, updated in place), followed by the readout, skip term
// and gate (paperlens tutorial "Mamba と状態空間モデル": recurrent inference
// at constant cost per token; ihouse article on Mamba-3: the SISO state
// update is an outer product with low, constant arithmetic intensity, so the
// step is bound by memory traffic).
//
// Layout: 4 consecutive lanes own one (b, d) and each holds 4 of its 16
// states as one float4, so a wave streams 16 channels = 1 KiB of contiguous
// state with 16-byte loads and stores.  The readout's 16-term sum is the
// lane's 4-term partial plus two cross-lane butterfly steps; lane 0 of the
// quad applies the skip term and gate and stores y.

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

template <typename IO> struct Quad;  // 4 consecutive B or C values
template <> struct Quad<float> {
  __device__ __forceinline__ static float4 load(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
};
template <> struct Quad<bf16> {
  __device__ __forceinline__ static float4 load(const bf16* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  }
};

__device__ __forceinline__ float zoh_update(float h, float av, float dv, float bv, float xv) {
  const float a = fast_exp2(dv * (av * kLog2e));  // Abar = exp(delta * A)
  const float bx = bv * xv;
  if (av != 0.0f) {
    const float q = bx * (1.0f / av);              // B x / A
    return __builtin_fmaf(a, h + q, -q);           // Abar (h + q) - q
  }
  return __builtin_fmaf(dv, bx, h);                // A == 0: Bbar = delta * B
}

template <typename IO>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t ch = gid >> 2;  // (b, d)
  const int q = (int)(gid & 3);
  if (ch >= a.batch * a.dim) return;  // whole quads leave together
  const int64_t b = ch / a.dim;
  const int d = (int)(ch % a.dim);

  float4* hp = reinterpret_cast<float4*>(a.h) + ch * 4 + q;
  float4 h = *hp;
  const float4 A = reinterpret_cast<const float4*>(a.A)[(size_t)d * 4 + q];
  const float4 Bq = Quad<IO>::load(static_cast<const IO*>(a.B) + b * kDState + 4 * q);
  const float4 Cq = Quad<IO>::load(static_cast<const IO*>(a.C) + b * kDState + 4 * q);
  const float xv = io<IO>::load(static_cast<const IO*>(a.x) + ch);
  const float dv = io<IO>::load(static_cast<const IO*>(a.delta) + ch);

  h.x = zoh_update(h.x, A.x, dv, Bq.x, xv);
  h.y = zoh_update(h.y, A.y, dv, Bq.y, xv);
  h.z = zoh_update(h.z, A.z, dv, Bq.z, xv);
  h.w = zoh_update(h.w, A.w, dv, Bq.w, xv);
  *hp = h;

  float p = Cq.x * h.x;
  p = __builtin_fmaf(Cq.y, h.y, p);
  p = __builtin_fmaf(Cq.z, h.z, p);
  p = __builtin_fmaf(Cq.w, h.w, p);
  p += __shfl_xor(p, 1);
  p += __shfl_xor(p, 2);
  if (q == 0) {
    const float Dd = a.Dskip ? a.Dskip[d] : 0.0f;
    const float pre = __builtin_fmaf(Dd, xv, p);
    const float yv = a.z ? pre * silu(io<IO>::load(static_cast<const IO*>(a.z) + ch)) : pre;
    io<IO>::store(static_cast<IO*>(a.y) + ch, yv);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool io_bf16, hipStream_t stream) {
  const int64_t threads = a.batch * a.dim * 4;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (io_bf16)
    hipLaunchKernelGGL(decode_step_kernel<bf16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_step_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ssm
