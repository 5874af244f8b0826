// ssm_decode.hip -- single-token recurrent decode step for gfx950 (wave64).
//
// One step of the scan's recurrence applied to a resident state
// h[b, d, 0:16] (fp32, updated in place), followed by the readout, skip term
// and gate (paperlens tutorial "Mamba と状態空間モデル": recurrent inference
// at constant cost per token; ihouse article on Mamba-3: the SISO state
// update is an outer product with low, constant arithmetic intensity, so the
// step is bound by memory traffic).
//
// Layout: L = N/4 consecutive lanes own one (b, d) and each holds 4 of its N
// states (N = 16, 32, 64, 128) as one float4, so a wave streams 1 KiB of
// contiguous state with 16-byte non-temporal loads and stores (the state is
// touched once per step).  The readout's N-term sum is the lane's 4-term
// partial plus DPP quad swaps, row half-mirror and mirror exchanges (and a
// 16-lane shuffle for N = 128); lane 0 of the channel applies the skip term
// and gate and stores y.  The grid's y dimension is the batch row, so no
// 64-bit division splits a flat index.  Variants (template bit V, as in the
// scan): A per channel (one exp and one coefficient per lane) and the Euler
// rule Bbar = delta * B.

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

typedef float v4f __attribute__((ext_vector_type(4)));

// Value of the lane `mask` places away inside each group of 4 lanes (DPP quad
// permutation; 0xB1 swaps neighbours, 0x4E swaps pairs).
template <int PERM>
__device__ __forceinline__ float quad_swap(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), PERM, 0xf, 0xf, false));
}

// One ZOH step of one state: h' = Abar*h + Bbar*x with Abar = exp(delta*A),
// Bbar*x = (Abar - 1) * (B*x/A) = fma(Abar, q, -q).  A zero step leaves h
// bit-for-bit unchanged; A == 0 takes the limit Bbar = delta*B.
__device__ __forceinline__ float zoh_update(float h, float av, float iav, float dl, float dv,
                                           float bx) {
  const float abar = fast_exp2(dl * av);  // dl = delta * log2(e)
  const float q = bx * iav;               // iav = 1/A
  const float b = av != 0.0f ? __builtin_fmaf(abar, q, -q) : dv * bx;
  return __builtin_fmaf(abar, h, b);
}

// Value of the lane that DPP control CTRL pairs with (row_half_mirror 0x141,
// row_mirror 0x140).
template <int CTRL>
__device__ __forceinline__ float row_swap(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Variant bits of the decode kernel (as in the scan): A given per channel,
// and the Euler rule Bbar = delta * B.
constexpr int kDecScalarA = 1;
constexpr int kDecEuler = 2;

// One step of one state for the variants: Abar = exp(delta * A) (a = Abar
// shared by the channel's states when A is per channel), coefficient k of B*x:
// (Abar - 1)/A for the hold (delta at A == 0), delta for Euler.
__device__ __forceinline__ float var_update(float h, float abar, float k, float bx) {
  return __builtin_fmaf(abar, h, k * bx);
}

// Batch rows per thread: each thread updates the same (channel, quarter) of
// kRows consecutive rows, so the channel's A and D are loaded once for all of
// them and kRows state loads are in flight per lane.
constexpr int kRows = 2;

template <typename IO, int N, int V>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  constexpr int L = N / 4;  // lanes per channel
  const int t = blockIdx.x * 256 + threadIdx.x;  // (channel, quarter) in one batch row
  const int d = t / L;
  const int q = t % L;
  if (d >= a.dim) return;  // a channel's lanes leave together
  const int64_t b0 = a.row0 + (int64_t)blockIdx.y * kRows;
  // rows of this block (block-uniform; fewer in the last block of a ragged batch)
  const int nr = (int)(a.batch - b0 < kRows ? a.batch - b0 : kRows);
  // Every load is issued before any result is waited on.  The small shared
  // and per-channel inputs go first and the streamed state (touched once per
  // step, so read and written non-temporally) last; on MI355X this order and
  // plain loads for x, delta and z measured fastest.
  v4f A;
  if constexpr (V & kDecScalarA) {
    const float ad = a.A[d];
    A = v4f{ad, ad, ad, ad};
  } else {
    A = reinterpret_cast<const v4f*>(a.A)[(size_t)d * L + q];
  }
  // optional inputs are read unconditionally (from a valid stand-in when
  // absent): a branch between loads makes the compiler wait for all of them
  const IO* zsrc = static_cast<const IO*>(a.z ? a.z : a.x);
  const float* dsrc = a.Dskip ? a.Dskip : a.A;
  float dload = dsrc[d];
  float4 Bq[kRows], Cq[kRows];
  float xv[kRows], dv[kRows], zv[kRows];
  v4f h[kRows];
  v4f* hp[kRows];
  size_t ch[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int64_t b = b0 + (r < nr ? r : 0);  // rows past the batch repeat row b0 (not stored)
    ch[r] = (size_t)b * a.dim + d;
    hp[r] = reinterpret_cast<v4f*>(a.h) + ch[r] * L + q;
    Bq[r] = Quad<IO>::load(static_cast<const IO*>(a.B) + b * N + 4 * q);
    Cq[r] = Quad<IO>::load(static_cast<const IO*>(a.C) + b * N + 4 * q);
    xv[r] = io<IO>::load(static_cast<const IO*>(a.x) + ch[r]);
    dv[r] = io<IO>::load(static_cast<const IO*>(a.delta) + ch[r]);
    zv[r] = io<IO>::load(zsrc + ch[r]);
  }
  asm volatile("" : "+v"(dload));  // keep the load here, unconditional
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    asm volatile("" : "+v"(zv[r]));
    h[r] = __builtin_nontemporal_load(hp[r]);
  }
  const float Dd = a.Dskip ? dload : 0.0f;
  v4f iA;
  if constexpr (V == 0) {
    iA = v4f{__builtin_amdgcn_rcpf(A.x), __builtin_amdgcn_rcpf(A.y), __builtin_amdgcn_rcpf(A.z),
             __builtin_amdgcn_rcpf(A.w)};
  }

#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    if (r >= nr) break;
    const float dl = dv[r] * kLog2e;
    v4f& hr = h[r];
    const float x = xv[r];
    if constexpr (V == 0) {
      hr.x = zoh_update(hr.x, A.x, iA.x, dl, dv[r], Bq[r].x * x);
      hr.y = zoh_update(hr.y, A.y, iA.y, dl, dv[r], Bq[r].y * x);
      hr.z = zoh_update(hr.z, A.z, iA.z, dl, dv[r], Bq[r].z * x);
      hr.w = zoh_update(hr.w, A.w, iA.w, dl, dv[r], Bq[r].w * x);
    } else if constexpr (V & kDecScalarA) {
      // one exp and one coefficient for the channel's states
      const float abar = fast_exp2(dl * A.x);
      const float k = (V & kDecEuler) ? dv[r]
                      : (A.x != 0.0f ? (abar - 1.0f) * __builtin_amdgcn_rcpf(A.x) : dv[r]);
      hr.x = var_update(hr.x, abar, k, Bq[r].x * x);
      hr.y = var_update(hr.y, abar, k, Bq[r].y * x);
      hr.z = var_update(hr.z, abar, k, Bq[r].z * x);
      hr.w = var_update(hr.w, abar, k, Bq[r].w * x);
    } else {  // Euler with A per state
      hr.x = var_update(hr.x, fast_exp2(dl * A.x), dv[r], Bq[r].x * x);
      hr.y = var_update(hr.y, fast_exp2(dl * A.y), dv[r], Bq[r].y * x);
      hr.z = var_update(hr.z, fast_exp2(dl * A.z), dv[r], Bq[r].z * x);
      hr.w = var_update(hr.w, fast_exp2(dl * A.w), dv[r], Bq[r].w * x);
    }
    __builtin_nontemporal_store(hr, hp[r]);

    float p = Cq[r].x * hr.x;
    p = __builtin_fmaf(Cq[r].y, hr.y, p);
    p = __builtin_fmaf(Cq[r].z, hr.z, p);
    p = __builtin_fmaf(Cq[r].w, hr.w, p);
    p += quad_swap<0xB1>(p);
    p += quad_swap<0x4E>(p);
    if constexpr (L >= 8) p += row_swap<0x141>(p);  // lanes i and 7 - i: the other quad
    if constexpr (L >= 16) p += row_swap<0x140>(p);  // lanes i and 15 - i: the other half row
    if constexpr (L >= 32) p += __shfl_xor(p, 16, kWave);
    if (q == 0) {
      const float pre = __builtin_fmaf(Dd, x, p);
      io<IO>::store(static_cast<IO*>(a.y) + ch[r], a.z ? pre * silu(zv[r]) : pre);
    }
  }
}

template <int N, int V>
hipError_t launch_decode_n(const DecodeArgs& args, bool io_bf16, hipStream_t stream) {
  const int64_t threads = (int64_t)args.dim * (N / 4);  // per batch row
  constexpr int64_t kMaxRows = 65535;              // rows per launch (grid y <= 65535)
  for (int64_t r0 = 0; r0 < args.batch; r0 += kMaxRows) {
    DecodeArgs a = args;
    a.row0 = r0;
    const int64_t rows = args.batch - r0 < kMaxRows ? args.batch - r0 : kMaxRows;
    a.batch = r0 + rows;  // last row (exclusive) of this launch
    const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)((rows + kRows - 1) / kRows));
    if (io_bf16)
      hipLaunchKernelGGL((decode_step_kernel<bf16, N, V>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_step_kernel<float, N, V>), grid, dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

namespace {
template <int V>
hipError_t launch_decode_v(const DecodeArgs& args, bool io_bf16, hipStream_t stream) {
  switch (args.dstate) {
    case 16: return launch_decode_n<16, V>(args, io_bf16, stream);
    case 32: return launch_decode_n<32, V>(args, io_bf16, stream);
    case 64: return launch_decode_n<64, V>(args, io_bf16, stream);
    case 128: return launch_decode_n<128, V>(args, io_bf16, stream);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_decode(const DecodeArgs& args, bool io_bf16, hipStream_t stream) {
  const int v = (args.a_per_channel ? kDecScalarA : 0) | (args.euler ? kDecEuler : 0);
  switch (v) {
    case 0: return launch_decode_v<0>(args, io_bf16, stream);
    case kDecScalarA: return launch_decode_v<kDecScalarA>(args, io_bf16, stream);
    case kDecEuler: return launch_decode_v<kDecEuler>(args, io_bf16, stream);
    default: return launch_decode_v<kDecScalarA | kDecEuler>(args, io_bf16, stream);
  }
}

}  // namespace ssm
