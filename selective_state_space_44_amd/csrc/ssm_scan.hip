// ssm_scan.hip -- selective scan forward kernels for gfx950 (wave64).
//
// Computes, per batch b, channel d, state n and step t (ultralytics glossary
// "State Space Models (SSM)", section "SSMの仕組み"; paperlens tutorial
// "Mamba と状態空間モデル", eq.(2) and the selection section):
//   Abar = exp(delta[b,t,d] * A[d,n]),  Bbar = (Abar - 1) / A[d,n] * B[b,t,n]
//   h    = Abar * h + Bbar * x[b,t,d]
//   y[b,t,d] = (sum_n C[b,t,n] h[n] + D[d] x[b,t,d]) * SiLU(z[b,t,d])
//
// Work decomposition (no MFMA: nothing here is a dense contraction).
//   * A block owns 64 consecutive channels of one batch row and one chunk of
//     the sequence.  Lane j of every wave holds channel d0 + j; the block has
//     G waves and wave g holds the NPL = 16/G state indices
//     n in [g*NPL, (g+1)*NPL) of those 64 channels.  The fp32 state lives in
//     VGPRs for the whole chunk and never touches HBM.
//   * B[b,t,n] and C[b,t,n] are the same for all 64 lanes of a wave, so they
//     are read with scalar loads and fed to the VALU as SGPR operands; x and
//     delta are read once per lane per step (one coalesced row segment per
//     wave) through a buffer resource whose row offset is a scalar, so the
//     inner loop does no per-lane address arithmetic.
//   * Update form: with q = B*x/A the ZOH step is h' = Abar*(h + q) - q,
//     i.e. one add and one fma per element after the exp2, with
//     Abar = exp2(delta * A*log2(e)).
//   * Readout: each wave forms its partial sum over its NPL states for every
//     step of a T-step tile, writes it to LDS, and after one barrier wave g
//     finishes steps s = g, g+G, ... of the tile: sum of the G partials (fixed
//     order, so results are deterministic), skip term, SiLU gate, and one
//     coalesced store of y.
//   * Sequence chunks (paperlens tutorial, parallel-scan section: the update
//     h_t = Abar_t h_{t-1} + u_t composes associatively): when the plan cuts
//     L into K chunks, a first kernel runs every chunk but the last from a
//     zero state and records its end state hloc_c and sum of delta; a carry
//     kernel composes the affine maps h -> P_c h + hloc_c with
//     P_c = exp(A * sum(delta over chunk c)) in chunk order; the main kernel
//     then runs every chunk from its true entering state.
//   * A == 0 (which the ZOH formula reaches only as a limit) switches the
//     affected wave to a form with that limit, Bbar = delta * B.

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

// Load NPL consecutive B (or C) values starting at a wave-uniform address.
template <typename IO, int NPL> struct BCLoad;
template <int NPL> struct BCLoad<float, NPL> {
  __device__ __forceinline__ static void load(const float* __restrict__ p, float (&out)[NPL]) {
#pragma unroll
    for (int k = 0; k < NPL; ++k) out[k] = p[k];
  }
};
template <int NPL> struct BCLoad<bf16, NPL> {
  __device__ __forceinline__ static void load(const bf16* __restrict__ p, float (&out)[NPL]) {
    if constexpr (NPL >= 2) {
      // NPL is even and the group start n0 is even: whole aligned dwords.
      const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
      for (int i = 0; i < NPL / 2; ++i) {
        uint32_t v = w[i];
        out[2 * i] = __uint_as_float(v << 16);
        out[2 * i + 1] = __uint_as_float(v & 0xffff0000u);
      }
    } else {
      uintptr_t addr = reinterpret_cast<uintptr_t>(p);
      uint32_t v = *reinterpret_cast<const uint32_t*>(addr & ~uintptr_t(3));
      out[0] = (addr & 2) ? __uint_as_float(v & 0xffff0000u) : __uint_as_float(v << 16);
    }
  }
};

// One ZOH step of NPL states of one channel.
template <int NPL, bool ZERO_A>
__device__ __forceinline__ void zoh_step(float dv, float xv, const float (&Bv)[NPL],
                                         const float (&A2)[NPL], const float (&iA)[NPL],
                                         float (&h)[NPL]) {
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const float a = fast_exp2(dv * A2[k]);  // Abar
    const float bx = Bv[k] * xv;
    if constexpr (!ZERO_A) {
      const float q = bx * iA[k];            // B x / A
      h[k] = __builtin_fmaf(a, h[k] + q, -q);
    } else {
      // (Abar - 1)/A, or its limit delta where A == 0 (iA is then +-inf).
      const bool lim = __builtin_isinf(iA[k]);
      const float w = lim ? dv : (a - 1.0f) * iA[k];
      h[k] = __builtin_fmaf(a, h[k], w * bx);
    }
  }
}

// Per-lane constants: A*log2(e) and 1/A for this wave's states.
template <int NPL>
__device__ __forceinline__ bool load_A(const float* __restrict__ A, int d, int n0,
                                       float (&A2)[NPL], float (&iA)[NPL]) {
  bool zero = false;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const float av = A[(size_t)d * kDState + n0 + k];
    A2[k] = av * kLog2e;
    iA[k] = 1.0f / av;
    zero |= (av == 0.0f);
  }
  return zero;
}

// Rows [t_begin, t_end) of one batch row of an [b, L, dim] tensor as a buffer.
template <typename IO>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const IO* p, int b, int64_t seqlen,
                                                            int dim, int64_t t_begin,
                                                            int64_t t_end) {
  const size_t first = ((size_t)b * seqlen + t_begin) * dim;
  return make_rsrc(p + first, (uint32_t)((size_t)(t_end - t_begin) * dim * sizeof(IO)));
}

struct Chunk {
  int lane, g, b, c, d;
  bool active;
  int64_t t_begin, t_end;
};

__device__ __forceinline__ Chunk chunk_coords(int dim, int64_t seqlen, int64_t chunk_len) {
  Chunk k;
  k.lane = threadIdx.x % kWave;
  k.g = wave_id();
  k.b = blockIdx.z;
  k.c = blockIdx.y;
  const int draw = blockIdx.x * kWave + k.lane;
  k.active = draw < dim;
  k.d = k.active ? draw : dim - 1;
  k.t_begin = (int64_t)k.c * chunk_len;
  k.t_end = min(seqlen, k.t_begin + chunk_len);
  return k;
}

// ---------------------------------------------------------------------------
// Main scan: one chunk of 64 channels x all 16 states per block.
// ---------------------------------------------------------------------------
template <typename IO, int G, int T, bool ZERO_A>
__device__ __forceinline__ void scan_chunk(
    const IO* __restrict__ x, const IO* __restrict__ delta, const IO* __restrict__ B,
    const IO* __restrict__ C, const IO* __restrict__ z, IO* __restrict__ y, float Dd,
    int64_t seqlen, int dim, const Chunk& k, float* part, const float (&A2)[kDState / G],
    const float (&iA)[kDState / G], float (&h)[kDState / G]) {
  constexpr int NPL = kDState / G;
  const int n0 = k.g * NPL;
  const __amdgpu_buffer_rsrc_t rx = rows_rsrc(x, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t rd = rows_rsrc(delta, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t rz = rows_rsrc(z ? z : x, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t ry = rows_rsrc(y, k.b, seqlen, dim, k.t_begin, k.t_end);
  const bool has_z = z != nullptr;
  const uint32_t voff = (uint32_t)k.d * sizeof(IO);
  const uint32_t row_bytes = (uint32_t)dim * sizeof(IO);
  const IO* Bp = B + ((size_t)k.b * seqlen + k.t_begin) * kDState + n0;
  const IO* Cp = C + ((size_t)k.b * seqlen + k.t_begin) * kDState + n0;
  const int nsteps = (int)(k.t_end - k.t_begin);

  int pbuf = 0;
  // Finish `ns` steps starting at local step s0 whose partial sums are in p.
  auto finish = [&](const float* p, int s0, int ns) {
    if constexpr (G == 1) {
      for (int s = 0; s < ns; ++s) {
        const uint32_t so = (uint32_t)(s0 + s) * row_bytes;
        const float pre = __builtin_fmaf(Dd, buf<IO>::load(rx, voff, so), p[s]);
        const float yv = has_z ? pre * silu(buf<IO>::load(rz, voff, so)) : pre;
        if (k.active) buf<IO>::store(yv, ry, voff, so);
      }
    } else {
      float* pb = part + pbuf * (G * T * kWave);
      for (int s = 0; s < ns; ++s) pb[(k.g * T + s) * kWave + k.lane] = p[s];
      __syncthreads();
      for (int s = k.g; s < ns; s += G) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < G; ++w) sum += pb[(w * T + s) * kWave + k.lane];
        const uint32_t so = (uint32_t)(s0 + s) * row_bytes;
        const float pre = __builtin_fmaf(Dd, buf<IO>::load(rx, voff, so), sum);
        const float yv = has_z ? pre * silu(buf<IO>::load(rz, voff, so)) : pre;
        if (k.active) buf<IO>::store(yv, ry, voff, so);
      }
      pbuf ^= 1;
    }
  };

  int s0 = 0;
  for (; s0 + T <= nsteps; s0 += T) {
    float xv[T], dv[T], p[T];
#pragma unroll
    for (int s = 0; s < T; ++s) {
      const uint32_t so = (uint32_t)(s0 + s) * row_bytes;
      xv[s] = buf<IO>::load(rx, voff, so);
      dv[s] = buf<IO>::load(rd, voff, so);
    }
#pragma unroll
    for (int s = 0; s < T; ++s) {
      float Bv[NPL], Cv[NPL];
      BCLoad<IO, NPL>::load(Bp + (size_t)(s0 + s) * kDState, Bv);
      BCLoad<IO, NPL>::load(Cp + (size_t)(s0 + s) * kDState, Cv);
      zoh_step<NPL, ZERO_A>(dv[s], xv[s], Bv, A2, iA, h);
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) acc = __builtin_fmaf(Cv[j], h[j], acc);
      p[s] = acc;
    }
    finish(p, s0, T);
  }
  // ragged end of the chunk: one step per tile
  for (; s0 < nsteps; ++s0) {
    const uint32_t so = (uint32_t)s0 * row_bytes;
    const float xs = buf<IO>::load(rx, voff, so);
    const float ds = buf<IO>::load(rd, voff, so);
    float Bv[NPL], Cv[NPL];
    BCLoad<IO, NPL>::load(Bp + (size_t)s0 * kDState, Bv);
    BCLoad<IO, NPL>::load(Cp + (size_t)s0 * kDState, Cv);
    zoh_step<NPL, ZERO_A>(ds, xs, Bv, A2, iA, h);
    float p[1] = {0.0f};
#pragma unroll
    for (int j = 0; j < NPL; ++j) p[0] = __builtin_fmaf(Cv[j], h[j], p[0]);
    finish(p, s0, 1);
  }
}

template <typename IO, int G, int T>
__global__ __launch_bounds__(kWave* G) void scan_fwd_kernel(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, const IO* __restrict__ C, const float* __restrict__ Dskip,
    const IO* __restrict__ z, const float* __restrict__ h0, IO* __restrict__ y,
    float* __restrict__ h_last, const float* __restrict__ ws_hin, int64_t seqlen,
    int64_t chunk_len, int dim, int nchunks) {
  constexpr int NPL = kDState / G;
  __shared__ float part[G > 1 ? 2 * G * T * kWave : 1];
  const Chunk k = chunk_coords(dim, seqlen, chunk_len);
  const int n0 = k.g * NPL;

  float A2[NPL], iA[NPL], h[NPL];
  const bool zero = load_A<NPL>(A, k.d, n0, A2, iA);
  const float* hinit = nullptr;
  if (nchunks > 1)
    hinit = ws_hin + (((size_t)k.b * nchunks + k.c) * dim + k.d) * kDState + n0;
  else if (h0)
    hinit = h0 + ((size_t)k.b * dim + k.d) * kDState + n0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) h[j] = hinit ? hinit[j] : 0.0f;
  const float Dd = Dskip ? Dskip[k.d] : 0.0f;

  if (__builtin_amdgcn_ballot_w64(zero) != 0)
    scan_chunk<IO, G, T, true>(x, delta, B, C, z, y, Dd, seqlen, dim, k, part, A2, iA, h);
  else
    scan_chunk<IO, G, T, false>(x, delta, B, C, z, y, Dd, seqlen, dim, k, part, A2, iA, h);

  if (k.c == nchunks - 1 && h_last && k.active) {
    float* hl = h_last + ((size_t)k.b * dim + k.d) * kDState + n0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) hl[j] = h[j];
  }
}

// ---------------------------------------------------------------------------
// Carry pass 1: end state of every chunk but the last, started from zero,
// plus the chunk's sum of delta (accumulated in fp64).
// ---------------------------------------------------------------------------
template <typename IO, int G, bool ZERO_A>
__device__ __forceinline__ void chunk_state(const IO* __restrict__ x,
                                            const IO* __restrict__ delta,
                                            const IO* __restrict__ B, int64_t seqlen, int dim,
                                            const Chunk& k, const float (&A2)[kDState / G],
                                            const float (&iA)[kDState / G],
                                            float (&h)[kDState / G], double& sd) {
  constexpr int NPL = kDState / G;
  constexpr int U = 8;
  const int n0 = k.g * NPL;
  const __amdgpu_buffer_rsrc_t rx = rows_rsrc(x, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t rd = rows_rsrc(delta, k.b, seqlen, dim, k.t_begin, k.t_end);
  const uint32_t voff = (uint32_t)k.d * sizeof(IO);
  const uint32_t row_bytes = (uint32_t)dim * sizeof(IO);
  const IO* Bp = B + ((size_t)k.b * seqlen + k.t_begin) * kDState + n0;
  const int nsteps = (int)(k.t_end - k.t_begin);
  int s0 = 0;
  for (; s0 + U <= nsteps; s0 += U) {
    float xv[U], dv[U];
#pragma unroll
    for (int s = 0; s < U; ++s) {
      const uint32_t so = (uint32_t)(s0 + s) * row_bytes;
      xv[s] = buf<IO>::load(rx, voff, so);
      dv[s] = buf<IO>::load(rd, voff, so);
    }
#pragma unroll
    for (int s = 0; s < U; ++s) {
      float Bv[NPL];
      BCLoad<IO, NPL>::load(Bp + (size_t)(s0 + s) * kDState, Bv);
      zoh_step<NPL, ZERO_A>(dv[s], xv[s], Bv, A2, iA, h);
      sd += (double)dv[s];
    }
  }
  for (; s0 < nsteps; ++s0) {
    const uint32_t so = (uint32_t)s0 * row_bytes;
    const float xs = buf<IO>::load(rx, voff, so);
    const float ds = buf<IO>::load(rd, voff, so);
    float Bv[NPL];
    BCLoad<IO, NPL>::load(Bp + (size_t)s0 * kDState, Bv);
    zoh_step<NPL, ZERO_A>(ds, xs, Bv, A2, iA, h);
    sd += (double)ds;
  }
}

template <typename IO, int G>
__global__ __launch_bounds__(kWave* G) void scan_chunk_state_kernel(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, float* __restrict__ ws_hloc, double* __restrict__ ws_sdelta,
    int64_t seqlen, int64_t chunk_len, int dim, int nchunks) {
  constexpr int NPL = kDState / G;
  const Chunk k = chunk_coords(dim, seqlen, chunk_len);  // k.c in [0, nchunks-2]
  const int n0 = k.g * NPL;
  float A2[NPL], iA[NPL], h[NPL];
  const bool zero = load_A<NPL>(A, k.d, n0, A2, iA);
#pragma unroll
  for (int j = 0; j < NPL; ++j) h[j] = 0.0f;
  double sd = 0.0;
  if (__builtin_amdgcn_ballot_w64(zero) != 0)
    chunk_state<IO, G, true>(x, delta, B, seqlen, dim, k, A2, iA, h, sd);
  else
    chunk_state<IO, G, false>(x, delta, B, seqlen, dim, k, A2, iA, h, sd);
  if (k.active) {
    const size_t cd = ((size_t)k.b * nchunks + k.c) * dim + k.d;
    float* hl = ws_hloc + cd * kDState + n0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) hl[j] = h[j];
    if (k.g == 0) ws_sdelta[cd] = sd;
  }
}

// ---------------------------------------------------------------------------
// Carry pass 2: compose h -> P_c h + hloc_c over the chunks in order and
// record the state entering every chunk.  One thread per (b, d, n).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scan_carry_kernel(
    const float* __restrict__ A, const float* __restrict__ h0,
    const float* __restrict__ ws_hloc, const double* __restrict__ ws_sdelta,
    float* __restrict__ ws_hin, int batch, int dim, int nchunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)batch * dim * kDState;
  if (i >= total) return;
  const int n = (int)(i % kDState);
  const int64_t bd = i / kDState;
  const int d = (int)(bd % dim);
  const int64_t b = bd / dim;
  const float A2 = A[(size_t)d * kDState + n] * kLog2e;
  float h = h0 ? h0[i] : 0.0f;
  for (int c = 0; c < nchunks; ++c) {
    const size_t cd = ((size_t)b * nchunks + c) * dim + d;
    ws_hin[cd * kDState + n] = h;
    if (c + 1 < nchunks) {
      const float P = fast_exp2((float)((double)A2 * ws_sdelta[cd]));
      h = __builtin_fmaf(P, h, ws_hloc[cd * kDState + n]);
    }
  }
}

__global__ __launch_bounds__(256) void copy_state_kernel(const float* __restrict__ h0,
                                                         float* __restrict__ h_last,
                                                         int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) h_last[i] = h0 ? h0[i] : 0.0f;
}

constexpr int tile_for(int G) { return G >= 8 ? G : 8; }

template <typename IO, int G>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t stream) {
  constexpr int T = tile_for(G);
  const IO* x = static_cast<const IO*>(a.x);
  const IO* delta = static_cast<const IO*>(a.delta);
  const IO* B = static_cast<const IO*>(a.B);
  const unsigned gx = (unsigned)((a.dim + kWave - 1) / kWave);
  if (a.nchunks > 1) {
    dim3 grid1(gx, (unsigned)(a.nchunks - 1), (unsigned)a.batch);
    hipLaunchKernelGGL((scan_chunk_state_kernel<IO, G>), grid1, dim3(kWave * G), 0, stream, x,
                       delta, a.A, B, a.ws_hloc, a.ws_sdelta, a.seqlen, a.chunk_len, a.dim,
                       a.nchunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = (int64_t)a.batch * a.dim * kDState;
    hipLaunchKernelGGL(scan_carry_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, a.A, a.h0, a.ws_hloc, a.ws_sdelta, a.ws_hin, a.batch, a.dim,
                       a.nchunks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(gx, (unsigned)a.nchunks, (unsigned)a.batch);
  hipLaunchKernelGGL((scan_fwd_kernel<IO, G, T>), grid, dim3(kWave * G), 0, stream, x, delta,
                     a.A, B, static_cast<const IO*>(a.C), a.Dskip,
                     static_cast<const IO*>(a.z), a.h0, static_cast<IO*>(a.y), a.h_last,
                     a.ws_hin, a.seqlen, a.chunk_len, a.dim, a.nchunks);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_scan_io(const ScanArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_scan_t<IO, 1>(a, stream);
    case 2: return launch_scan_t<IO, 2>(a, stream);
    case 4: return launch_scan_t<IO, 4>(a, stream);
    case 8: return launch_scan_t<IO, 8>(a, stream);
    case 16: return launch_scan_t<IO, 16>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

ScanWorkspace scan_workspace_layout(int64_t batch, int64_t dim, int nchunks) {
  ScanWorkspace w{0, 0, 0, 0};
  if (nchunks <= 1) return w;
  auto align = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t states = (size_t)batch * nchunks * dim * kDState;
  w.hloc_off = 0;
  w.hin_off = align(states * sizeof(float));
  w.sdelta_off = w.hin_off + align(states * sizeof(float));
  w.total = w.sdelta_off + align((size_t)batch * nchunks * dim * sizeof(double));
  return w;
}

hipError_t launch_scan(const ScanArgs& a, bool io_bf16, int waves_per_group,
                       hipStream_t stream) {
  return io_bf16 ? launch_scan_io<bf16>(a, waves_per_group, stream)
                 : launch_scan_io<float>(a, waves_per_group, stream);
}

hipError_t launch_copy_state(const float* h0, float* h_last, int64_t count,
                             hipStream_t stream) {
  hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     stream, h0, h_last, count);
  return hipGetLastError();
}

}  // namespace ssm
