// ssm_scan_wide.hip -- selective scan for state sizes 32, 64 and 128 (gfx950,
// wave64).
//
// The same recurrence as ssm_scan.hip (zero-order hold or the Euler rule, A
// per (channel, state) or per channel; paperlens tutorial, eq. (2) and the
// selection section), for the larger states the pages mention (P1's d_state
// setting; the ihouse article's Mamba-3 runs at state size 128).  With more
// states per channel there are more waves per 64-channel group (8 or 16), so
// one pass over the whole sequence already puts 8-16 waves on each group and
// the chunked carry of the 16-state kernels is not needed:
//
//   block = 64 channels (one per lane) x G waves, wave g holds states
//   [g * N / G, (g + 1) * N / G) of its lane's channel in VGPRs (4 or 8);
//   8-step tiles of x, delta, z (fp32 [step][channel]) and B, C (fp32
//   [step][state]) are staged in LDS by the whole block; each wave adds its
//   states' part of C.h to an LDS partial, and after one barrier waves
//   0..7 finish one step each (sum of the G partials, D x, gate, store).
//
// Steps past the end of the sequence and channels past dim are staged as
// zeros, which are identities of the recurrence (Abar = 1, input term 0).
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

constexpr int kWT = 8;               // steps per tile
constexpr int kWideScalarA = 1;      // A is [dim]
constexpr int kWideEuler = 2;        // Bbar = delta * B

template <int N, int G>
struct WideSmem {
  float x[kWT][kWave];
  float dl[kWT][kWave];
  float z[kWT][kWave];
  float b[kWT][N];
  float c[kWT][N];
  float part[G][kWT][kWave];
};

__device__ __forceinline__ void pin_w(float& v) { asm volatile("" : "+v"(v)); }

// Input term Bbar * x from Abar, delta, 1/A and B x.
template <int V, bool ZERO_A>
__device__ __forceinline__ float wide_input(float a, float dv, float iA, float bx) {
  if constexpr ((V & kWideEuler) != 0) {
    return dv * bx;
  } else if constexpr (ZERO_A) {
    return (__builtin_isinf(iA) ? dv : (a - 1.0f) * iA) * bx;
  } else {
    const float q = bx * iA;
    return __builtin_fmaf(a, q, -q);
  }
}

template <typename IO, int N, int G, bool HAS_Z, int V, bool ZERO_A>
__device__ __forceinline__ void wide_body(WideSmem<N, G>& sm, const IO* __restrict__ x,
                                          const IO* __restrict__ delta,
                                          const IO* __restrict__ B, const IO* __restrict__ C,
                                          const IO* __restrict__ z, IO* __restrict__ y,
                                          const float (&A2)[N / G], const float (&iA)[N / G],
                                          float Dd, float (&h)[N / G], int b, int d0, int dim,
                                          int64_t seqlen) {
  constexpr int NPL = N / G;
  const int lane = threadIdx.x % kWave;
  const int g = wave_id();
  const int n0 = g * NPL;
  const int d = d0 + lane;
  for (int64_t t0 = 0; t0 < seqlen; t0 += kWT) {
    __syncthreads();  // the previous tile's epilogue has read the stage
    for (int i = threadIdx.x; i < kWT * kWave; i += kWave * G) {
      const int s = i / kWave, ch = i % kWave;
      const int64_t t = t0 + s;
      const bool ok = t < seqlen && d0 + ch < dim;
      const size_t off = ((size_t)b * seqlen + (ok ? t : 0)) * dim + (ok ? d0 + ch : 0);
      sm.x[s][ch] = ok ? io<IO>::load(x + off) : 0.0f;
      sm.dl[s][ch] = ok ? io<IO>::load(delta + off) : 0.0f;
      if constexpr (HAS_Z) sm.z[s][ch] = ok ? io<IO>::load(z + off) : 0.0f;
    }
    for (int i = threadIdx.x; i < kWT * N; i += kWave * G) {
      const int s = i / N, n = i % N;
      const int64_t t = t0 + s;
      const bool ok = t < seqlen;
      const size_t off = ((size_t)b * seqlen + (ok ? t : 0)) * N + n;
      sm.b[s][n] = ok ? io<IO>::load(B + off) : 0.0f;
      sm.c[s][n] = ok ? io<IO>::load(C + off) : 0.0f;
    }
    __syncthreads();
    // two steps per iteration: fully unrolled, the 8 states per lane of the
    // 128-state kernels spill (registers hold several steps' exponentials)
#pragma unroll 2
    for (int s = 0; s < kWT; ++s) {
      const float xv = sm.x[s][lane], dv = sm.dl[s][lane];
      float acc = 0.0f;
#pragma unroll
      for (int q = 0; q < NPL / 4; ++q) {
        const float4 b4 = reinterpret_cast<const float4*>(&sm.b[s][n0])[q];
        const float4 c4 = reinterpret_cast<const float4*>(&sm.c[s][n0])[q];
        const float bq[4] = {b4.x, b4.y, b4.z, b4.w};
        const float cq[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = 4 * q + j;
          const float a = fast_exp2(dv * A2[n]);
          h[n] = __builtin_fmaf(a, h[n], wide_input<V, ZERO_A>(a, dv, iA[n], bq[j] * xv));
          pin_w(h[n]);
          acc = __builtin_fmaf(cq[j], h[n], acc);
        }
      }
      sm.part[g][s][lane] = acc;
    }
    __syncthreads();
    for (int s = g; s < kWT; s += G) {
      const int64_t t = t0 + s;
      if (t >= seqlen || d >= dim) continue;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < G; ++w) sum += sm.part[w][s][lane];
      const float pre = __builtin_fmaf(Dd, sm.x[s][lane], sum);
      const size_t off = ((size_t)b * seqlen + t) * dim + d;
      if constexpr (HAS_Z)
        io<IO>::store(y + off, pre * silu(sm.z[s][lane]));
      else
        io<IO>::store(y + off, pre);
    }
  }
}

template <typename IO, int N, int G, bool HAS_Z, int V>
__global__ __launch_bounds__(kWave* G) void scan_wide_kernel(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, const IO* __restrict__ C, const float* __restrict__ Dskip,
    const IO* __restrict__ z, const float* __restrict__ h0, IO* __restrict__ y,
    float* __restrict__ h_last, int64_t seqlen, int dim) {
  constexpr int NPL = N / G;
  static_assert(NPL % 4 == 0, "b128 LDS reads of B and C");
  __shared__ WideSmem<N, G> sm;
  const int lane = threadIdx.x % kWave;
  const int g = wave_id();
  const int b = blockIdx.z;
  const int d0 = blockIdx.x * kWave;
  const bool active = d0 + lane < dim;
  const int d = active ? d0 + lane : dim - 1;
  const int n0 = g * NPL;
  float A2[NPL], iA[NPL], h[NPL];
  bool zero = false;
#pragma unroll
  for (int n = 0; n < NPL; ++n) {
    const float av = (V & kWideScalarA) ? A[d] : A[(size_t)d * N + n0 + n];
    A2[n] = av * kLog2e;
    iA[n] = 1.0f / av;
    zero |= av == 0.0f;
  }
  const size_t sidx = ((size_t)b * dim + d) * N + n0;
#pragma unroll
  for (int n = 0; n < NPL; ++n) h[n] = h0 ? h0[sidx + n] : 0.0f;
  const float Dd = Dskip ? Dskip[d] : 0.0f;
  if (__builtin_amdgcn_ballot_w64(zero) != 0)
    wide_body<IO, N, G, HAS_Z, V, true>(sm, x, delta, B, C, z, y, A2, iA, Dd, h, b, d0, dim,
                                        seqlen);
  else
    wide_body<IO, N, G, HAS_Z, V, false>(sm, x, delta, B, C, z, y, A2, iA, Dd, h, b, d0, dim,
                                         seqlen);
  if (h_last && active) {
#pragma unroll
    for (int n = 0; n < NPL; ++n) h_last[sidx + n] = h[n];
  }
}

template <typename IO, int N, int G, int V>
hipError_t launch_wide_t(const ScanArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.dim + kWave - 1) / kWave), 1, (unsigned)a.batch);
  const IO* x = static_cast<const IO*>(a.x);
  const IO* delta = static_cast<const IO*>(a.delta);
  const IO* B = static_cast<const IO*>(a.B);
  const IO* C = static_cast<const IO*>(a.C);
  const IO* z = static_cast<const IO*>(a.z);
  IO* y = static_cast<IO*>(a.y);
  if (a.z)
    hipLaunchKernelGGL((scan_wide_kernel<IO, N, G, true, V>), grid, dim3(kWave * G), 0, stream,
                       x, delta, a.A, B, C, a.Dskip, z, a.h0, y, a.h_last, a.seqlen, a.dim);
  else
    hipLaunchKernelGGL((scan_wide_kernel<IO, N, G, false, V>), grid, dim3(kWave * G), 0, stream,
                       x, delta, a.A, B, C, a.Dskip, z, a.h0, y, a.h_last, a.seqlen, a.dim);
  return hipGetLastError();
}

template <typename IO, int V>
hipError_t launch_wide_v(const ScanArgs& a, int dstate, hipStream_t stream) {
  switch (dstate) {
    case 32: return launch_wide_t<IO, 32, 8, V>(a, stream);    // 4 states per lane
    case 64: return launch_wide_t<IO, 64, 16, V>(a, stream);   // 4 states per lane
    case 128: return launch_wide_t<IO, 128, 16, V>(a, stream); // 8 states per lane
  }
  return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_wide_io(const ScanArgs& a, int dstate, hipStream_t stream) {
  const int V = (a.a_per_channel ? kWideScalarA : 0) | (a.euler ? kWideEuler : 0);
  switch (V) {
    case 0: return launch_wide_v<IO, 0>(a, dstate, stream);
    case kWideScalarA: return launch_wide_v<IO, kWideScalarA>(a, dstate, stream);
    case kWideEuler: return launch_wide_v<IO, kWideEuler>(a, dstate, stream);
    default: return launch_wide_v<IO, kWideScalarA | kWideEuler>(a, dstate, stream);
  }
}

}  // namespace

bool scan_wide_supported(int64_t dstate) {
  return dstate == 32 || dstate == 64 || dstate == 128;
}

hipError_t launch_scan_wide(const ScanArgs& a, int dstate, bool io_bf16, hipStream_t stream) {
  return io_bf16 ? launch_wide_io<bf16>(a, dstate, stream)
                 : launch_wide_io<float>(a, dstate, stream);
}

}  // namespace ssm
