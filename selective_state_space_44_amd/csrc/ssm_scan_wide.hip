// ssm_scan_wide.hip -- selective scan for state sizes 32, 64 and 128 (gfx950,
// wave64).
//
// The same recurrence as ssm_scan.hip (zero-order hold or the Euler rule, A
// per (channel, state) or per channel; paperlens tutorial, eq. (2) and the
// selection section), for the larger states the pages mention (P1's d_state
// setting; the ihouse article's Mamba-3 runs at state size 128).  With N
// states per channel there is enough work per channel group to fill the chip
// in one pass over the sequence, without the chunked carry of the 16-state
// kernels -- provided the blocks are small enough to balance over the CUs:
//
//   block = 16 channels x G waves (G = 4, 4, 8 for N = 32, 64, 128); lane l
//   holds channel l / 4 and quarter q = l % 4; wave g and quarter q own the
//   NPL = N / (4 G) states [(4 g + q) NPL, (4 g + q + 1) NPL) of the channel,
//   in VGPRs.  At the Mamba-2.8B shape that is 1280 blocks (5 per CU).
//   8-step tiles of x, delta, z ([step][channel]) and B, C ([step][state])
//   are staged in LDS two buffers deep: the global loads of tile i + 1 are
//   issued before tile i is computed and written to the other buffer after
//   it.  Each step's readout is summed over the 4 quarters with two DPP quad
//   swaps and over the G waves through LDS; after the tile's barrier the
//   first 128 threads finish one (step, channel) each (sum, D x, gate, store).
//
// Steps past the end of the sequence and channels past dim are staged as
// zeros, which are identities of the recurrence (Abar = 1, input term 0).
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

constexpr int kWT = 8;               // steps per tile
constexpr int kWQ = 4;               // lanes (quarters) per channel
constexpr int kWCh = kWave / kWQ;    // channels per block
// Waves per block (the states per lane follow: N / (4 G)).  Measured at
// (4, 4096, 5120) bf16: N = 32 with 4 waves (2 states per lane) 1.42 ms
// against 1.67 ms with 2; N = 64 with 4 waves (4 states) 1.92 ms against
// 2.47 (2 waves) and 2.49 (8 waves); N = 128 with 8 waves (4 states)
// 3.30 ms against 4.14 ms with 4.
constexpr int kWideG32 = 4;
constexpr int kWideG64 = 4;
constexpr int kWideG128 = 8;
constexpr int kWideScalarA = 1;      // A is [dim]
constexpr int kWideEuler = 2;        // Bbar = delta * B

template <int N, int G>
struct WideSmem {
  float x[2][kWT][kWCh];
  float dl[2][kWT][kWCh];
  float z[2][kWT][kWCh];
  float b[2][kWT][N];
  float c[2][kWT][N];
  float part[G][kWT][kWCh];
};

__device__ __forceinline__ void pin_w(float& v) { asm volatile("" : "+v"(v)); }

// Value of the lane that quad permutation PERM selects (0xB1 swaps
// neighbours, 0x4E swaps pairs).
template <int PERM>
__device__ __forceinline__ float quad_w(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), PERM, 0xf, 0xf, false));
}

// NPL consecutive floats of an LDS row with b64 / b128 reads.
template <int NPL>
__device__ __forceinline__ void read_row_w(const float* p, float (&out)[NPL]) {
  if constexpr (NPL == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    out[0] = v.x;
    out[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(p)[q];
      out[4 * q] = v.x;
      out[4 * q + 1] = v.y;
      out[4 * q + 2] = v.z;
      out[4 * q + 3] = v.w;
    }
  }
}

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
                                          const float* __restrict__ Dskip,
                                          const float (&A2)[N / (kWQ * G)],
                                          const float (&iA)[N / (kWQ * G)],
                                          float (&h)[N / (kWQ * G)], int b, int d0, int dim,
                                          int64_t seqlen) {
  constexpr int NPL = N / (kWQ * G);
  constexpr int BC = kWT * N / (kWave * G);  // B (and C) values per thread per tile
  static_assert(BC >= 1 && (kWT * N) % (kWave * G) == 0, "B/C tile splits over the block");
  static_assert(kWave * G >= kWT * kWCh, "x, delta, z tile: one value per thread");
  const int lane = threadIdx.x % kWave;
  const int g = wave_id();
  const int ch = lane / kWQ, q = lane % kWQ;
  const int n0 = (g * kWQ + q) * NPL;
  const int tid = threadIdx.x;
  // staging share: x, delta, z of one (step, channel) for the first 128
  // threads; BC values of B and C for every thread
  const int xs = tid / kWCh, xc = tid % kWCh;
  const bool xthr = tid < kWT * kWCh;
  float rx = 0.0f, rdl = 0.0f, rz = 0.0f, rb[BC], rc[BC];
  auto fetch = [&](int64_t t0) {
    if (xthr) {
      const int64_t t = t0 + xs;
      const bool ok = t < seqlen && d0 + xc < dim;
      const size_t off = ((size_t)b * seqlen + (ok ? t : 0)) * dim + (ok ? d0 + xc : 0);
      rx = ok ? io<IO>::load(x + off) : 0.0f;
      rdl = ok ? io<IO>::load(delta + off) : 0.0f;
      if constexpr (HAS_Z) rz = ok ? io<IO>::load(z + off) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < BC; ++k) {
      const int i = tid + k * kWave * G;
      const int64_t t = t0 + i / N;
      const bool ok = t < seqlen;
      const size_t off = ((size_t)b * seqlen + (ok ? t : 0)) * N + i % N;
      rb[k] = ok ? io<IO>::load(B + off) : 0.0f;
      rc[k] = ok ? io<IO>::load(C + off) : 0.0f;
    }
  };
  auto put = [&](int buf) {
    if (xthr) {
      sm.x[buf][xs][xc] = rx;
      sm.dl[buf][xs][xc] = rdl;
      if constexpr (HAS_Z) sm.z[buf][xs][xc] = rz;
    }
#pragma unroll
    for (int k = 0; k < BC; ++k) {
      const int i = tid + k * kWave * G;
      sm.b[buf][i / N][i % N] = rb[k];
      sm.c[buf][i / N][i % N] = rc[k];
    }
  };
  const int64_t ntiles = (seqlen + kWT - 1) / kWT;
  fetch(0);
  put(0);
  __syncthreads();
  for (int64_t it = 0; it < ntiles; ++it) {
    const int cur = (int)(it & 1);
    const int64_t t0 = it * kWT;
    if (it + 1 < ntiles) fetch(t0 + kWT);  // in flight during this tile
#pragma unroll 2
    for (int s = 0; s < kWT; ++s) {
      const float xv = sm.x[cur][s][ch], dv = sm.dl[cur][s][ch];
      float bn[NPL], cn[NPL];
      read_row_w<NPL>(&sm.b[cur][s][n0], bn);
      read_row_w<NPL>(&sm.c[cur][s][n0], cn);
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const float a = fast_exp2(dv * A2[j]);
        h[j] = __builtin_fmaf(a, h[j], wide_input<V, ZERO_A>(a, dv, iA[j], bn[j] * xv));
        pin_w(h[j]);
        acc = __builtin_fmaf(cn[j], h[j], acc);
      }
      acc += quad_w<0xB1>(acc);
      acc += quad_w<0x4E>(acc);
      if (q == 0) sm.part[g][s][ch] = acc;
    }
    __syncthreads();
    if (xthr) {
      const int64_t t = t0 + xs;
      const int d = d0 + xc;
      if (t < seqlen && d < dim) {
        float sum = sm.part[0][xs][xc];
#pragma unroll
        for (int w = 1; w < G; ++w) sum += sm.part[w][xs][xc];
        const float dd = Dskip ? Dskip[d] : 0.0f;
        const float pre = __builtin_fmaf(dd, sm.x[cur][xs][xc], sum);
        const size_t off = ((size_t)b * seqlen + t) * dim + d;
        if constexpr (HAS_Z)
          io<IO>::store(y + off, pre * silu(sm.z[cur][xs][xc]));
        else
          io<IO>::store(y + off, pre);
      }
    }
    if (it + 1 < ntiles) put(cur ^ 1);
    __syncthreads();
  }
}

template <typename IO, int N, int G, bool HAS_Z, int V>
__global__ __launch_bounds__(kWave* G) void scan_wide_kernel(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, const IO* __restrict__ C, const float* __restrict__ Dskip,
    const IO* __restrict__ z, const float* __restrict__ h0, IO* __restrict__ y,
    float* __restrict__ h_last, int64_t seqlen, int dim) {
  constexpr int NPL = N / (kWQ * G);
  __shared__ WideSmem<N, G> sm;
  const int lane = threadIdx.x % kWave;
  const int g = wave_id();
  const int b = blockIdx.z;
  const int d0 = blockIdx.x * kWCh;
  const int ch = lane / kWQ, q = lane % kWQ;
  const bool active = d0 + ch < dim;
  const int d = active ? d0 + ch : dim - 1;
  const int n0 = (g * kWQ + q) * NPL;
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
  if (__builtin_amdgcn_ballot_w64(zero) != 0)
    wide_body<IO, N, G, HAS_Z, V, true>(sm, x, delta, B, C, z, y, Dskip, A2, iA, h, b, d0, dim,
                                     seqlen);
  else
    wide_body<IO, N, G, HAS_Z, V, false>(sm, x, delta, B, C, z, y, Dskip, A2, iA, h, b, d0, dim,
                                      seqlen);
  if (h_last && active) {
#pragma unroll
    for (int n = 0; n < NPL; ++n) h_last[sidx + n] = h[n];
  }
}

template <typename IO, int N, int G, int V>
hipError_t launch_wide_t(const ScanArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.dim + kWCh - 1) / kWCh), 1, (unsigned)a.batch);
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
    case 32: return launch_wide_t<IO, 32, kWideG32, V>(a, stream);
    case 64: return launch_wide_t<IO, 64, kWideG64, V>(a, stream);
    case 128: return launch_wide_t<IO, 128, kWideG128, V>(a, stream);
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
