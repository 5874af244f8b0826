// ssm_ssd_bwd.hip -- backward of the per-head scan (step and decay shared by
// each head of 64 channels) in its masked-matrix form, every 32-step chunk
// independent, on the matrix cores.
//
// Method: the same sources as the forward (ihouse article on Mamba-3, section
// on Mamba's evolution: with A scalar the SSM is masked matrix products;
// paperlens tutorial, section on the parallel scan: chunks compose through
// their entering states).  Per head, with the state h_t an N x 64 matrix,
//   h_t = a_t h_{t-1} + coef_t B_t x_t^T,  pre_t = h_t^T C_t + D x_t,
//   y_t = pre_t SiLU(z_t),
// the adjoint g_t = dL/dh_t obeys g_{t-1} = a_t g_t + C_{t-1} dpre_{t-1}^T
// (g at the last step = C dpre^T + dh_last), and the gradients are
//   dx_t = coef_t u_t + D dpre_t          with u_t = g_t^T B_t,
//   dB_t = coef_t g_t x_t,  dC_t = h_t dpre_t,
//   dlog a_t = <g_t, a_t h_{t-1}> =: kappa_t,
//   dcoef_t = u_t . x_t,
// ddt_t = kappa_t A + dcoef_t dcoef/ddt and dA = sum_t kappa_t dt_t +
// dcoef_t dcoef/dA.  kappa needs no state per step: splitting g_t and
// a_t h_{t-1} of a chunk into their in-chunk and boundary parts,
//   kappa_t = sum_{i>=t, j<t} R_ij + sum_{i>=t} alpha_i + sum_{j<t} beta_j
//             + gamma
// with R = P o G (P, G below), alpha_i = ein_i dpre_i . (h_in^T C_i),
// beta_j = eout_j coef_j x_j . (g_out^T B_j), gamma = exp(s_last) <g_out,
// h_in>; the corner sum of the lower-triangular R is the exclusive prefix
// sum of (column sum - row sum).  Every term is a product of the size of
// kappa itself, so the split-bf16 products keep their relative accuracy.
//
// Passes (all chunks of 32 steps):
//   A, B  two walks over the chunks in one launch: forward from h0, storing
//      hbuf[c] = state entering chunk c; backward from dh_last, storing
//      gbuf[c] = adjoint leaving chunk c, and dh0;
//   C  per (head group, chunk, batch row): the chunk's gradients from hbuf[c]
//      and gbuf[c] (below): dx, dz, ddt, dA's and D's partial sums, dB and
//      dC summed over the group's heads;
//   D  the sums of dB, dC over head groups, of dA and dD over (batch row,
//      chunk).
// Chunk c of one head, steps i, j in 0..31, s_i = log decay from the chunk's
// start through step i, E_ij = exp(s_i - s_j) for j <= i (0 above), ein_i =
// exp(s_i), eout_j = exp(s_last - s_j), M = C B^T, G = dpre x^T:
//   ys = (E o M o coef_j) x + ein o (C h_in)          [32 x 64]  (= P x + ...)
//   u  = (E o M)^T dpre     + eout o (B g_out)         [32 x 64]
//   dB = coef o ((E o G)^T C + eout o (x g_out^T))     [32 x N]
//   dC = (E o G o coef_j) B + ein o (dpre h_in^T)      [32 x N]
// Precision as in the forward: B, C, x are exact bf16 operands; fp32 operands
// (states, dpre, the masked matrices) are split into bf16 high and low parts
// and the products of the significant pairs are summed in fp32.

#include "ssm_device.h"
#include "ssm_launch.h"
#include "ssm_mfma.h"

namespace ssm {
namespace {

constexpr int kQ = 32;        // steps per chunk
constexpr int kHD = 64;       // channels per head
constexpr int kRowP = kHD + 8;  // bf16 per staged row of 64 channels
constexpr int kRowT = kQ + 8;   // bf16 per row of a 32 x 32 matrix
constexpr int kThreads = 256;

// Eight bf16 values of one LDS column (rows 0..7 from p, stride in elements)
// as an MFMA operand: slot s = row s.
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ u32x4_t lds_col8(const uint16_t* p, int stride) {
  // element-wise into a 16-bit vector: 16-bit loads into register halves
  u16x8_t v;
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = p[s * stride];
  return __builtin_bit_cast(u32x4_t, v);
}

// Eight fp32 values as bf16 high and low operands.
__device__ __forceinline__ void split8(const float (&v)[8], u32x4_t& hi, u32x4_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) split_bf16(v[2 * m], v[2 * m + 1], h[m], l[m]);
  hi = {h[0], h[1], h[2], h[3]};
  lo = {l[0], l[1], l[2], l[3]};
}

__device__ __forceinline__ float bf16_at(const uint16_t* p) { return bf16_bits_to_f32(*p); }

__device__ __forceinline__ float sigmoid_f(float v) { return 1.0f / (1.0f + __expf(-v)); }

// bf16 bits of dt of step `lane` of a chunk for head h (0 past the sequence
// and for lanes >= 32).
__device__ __forceinline__ uint32_t load_dt(const void* dt, int64_t b, int64_t L, int64_t t0,
                                            int rows, int H, int h, int lane) {
  const __amdgpu_buffer_rsrc_t rsd =
      make_rsrc(static_cast<const uint16_t*>(dt) + (b * L + t0) * H, (uint32_t)rows * H * 2u);
  return lane < kQ ? __builtin_amdgcn_raw_buffer_load_b16(rsd, (uint32_t)(lane * H + h) * 2u, 0, 0)
                   : 0u;
}

// Per-step values of one head's chunk, from lanes < 32 of one wave, given
// the dt bits of step `lane` (load_dt): s2 (log2 decay from the chunk's start
// through the step), coef, and where given ein, eout and dt itself.  Returns
// the chunk's log2 decay (all lanes).
__device__ __forceinline__ float chunk_steps_raw(uint32_t raw, float Ah, bool coef_is_dt,
                                                 int lane, float* s2, float* coef, float* ein,
                                                 float* eout, float* dts) {
  const float dtv = bf16_bits_to_f32(raw);
  float s = dtv * Ah * kLog2e;
#pragma unroll
  for (int o = 1; o < kQ; o <<= 1) {
    const float v = __shfl_up(s, o);
    if (lane >= o) s += v;
  }
  const float last = __shfl(s, kQ - 1);
  if (lane < kQ) {
    s2[lane] = s;
    coef[lane] = coef_is_dt ? dtv : expm1f(dtv * Ah) / Ah;
    if (ein) ein[lane] = fast_exp2(s);
    if (eout) eout[lane] = fast_exp2(last - s);
    if (dts) dts[lane] = dtv;
  }
  return last;
}

// The same, loading dt.
__device__ __forceinline__ float chunk_steps(const void* dt, int64_t b, int64_t L, int64_t t0,
                                             int rows, int H, int h, float Ah, bool coef_is_dt,
                                             int lane, float* s2, float* coef, float* ein,
                                             float* eout, float* dts = nullptr) {
  return chunk_steps_raw(load_dt(dt, b, L, t0, rows, H, h, lane), Ah, coef_is_dt, lane, s2, coef,
                         ein, eout, dts);
}

// ---------------------------------------------------------------------------
// passes A and B: the two walks, one launch.  Blocks [0, 2H) walk forward:
// one per (half head, batch row), the state h (N states x 32 channels) in
// MFMA accumulators from h0, stored as the state entering each chunk, then
//   h <- exp(s_last) h + sum_t exp(s_last - s_t) coef_t B_t x_t^T.
// Blocks [2H, 4H) walk backward from dh_last with the adjoint g, stored as
// the adjoint leaving each chunk, then
//   g <- exp(s_last) g + sum_t exp(s_t) C_t dpre_t^T,
// and what reaches the start is dh0.  Both are chains of 32-step chunks
// (latency-bound, 2H blocks per batch row each), so they run side by side.
// Waves: (channel tile pt, state half nh); the next chunk's inputs are
// loaded while the current one is computed.
// ---------------------------------------------------------------------------
constexpr int kBC = 32;          // channels per block (half a head)
constexpr int kRowX = kBC + 8;   // bf16 per staged row of 32 channels

template <int N>
struct WalkSmem {
  alignas(16) uint16_t ms[kQ][N + 8];  // B (forward) or C (backward), [t][n]
  alignas(16) uint16_t eh[kQ][kRowX];  // weighted x or dpre, high part, [t][p]
  alignas(16) uint16_t el[kQ][kRowX];  // low part
  alignas(16) float s2[kQ], coef[kQ], ein[kQ], eout[kQ];
};

template <int N, bool HAS_Z, bool EULER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5)))
void ssd_bwd_walk_kernel(SsdBwdArgs a) {
  constexpr int NB = N / 8, NBV = NB / 8;
  constexpr int NT2 = N / 32;  // 16-state tiles per wave
  __shared__ WalkSmem<N> sm;
  const int H = a.nheads;
  const bool fwd = (int)blockIdx.x < 2 * H;
  const int bx = fwd ? (int)blockIdx.x : (int)blockIdx.x - 2 * H;
  const int h = bx >> 1, half = bx & 1;
  const int64_t b = blockIdx.y;
  const int dim = a.dim, K = a.nchunks;
  const int64_t L = a.seqlen;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int pt = w & 1, nh = w >> 1;
  const int ts = tid & (kQ - 1), cg = tid >> 5;  // staging: step, column group
  const int cb = h * kHD + kBC * half;           // first channel of the block
  const int d = cb + 16 * pt + r16;              // this lane's channel (result column)
  const float Ah = a.A[h];
  const size_t soff = (size_t)16 * nh * NT2 + 4 * g;  // this lane's first state
  const void* mat_in = fwd ? a.B : a.C;
  float* const out = fwd ? a.hbuf : a.gbuf;

  f32x4_t acc[NT2];
  {
    const float* init = fwd ? a.h0 : a.dh_last;
    const float* src = init ? init + ((size_t)b * dim + d) * N + soff : nullptr;
#pragma unroll
    for (int j = 0; j < NT2; ++j)
      acc[j] = src ? *reinterpret_cast<const f32x4_t*>(src + 16 * j) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // staging registers of one chunk: B or C (states NB cg .. + NB - 1 of step
  // ts); x, or dy and z (channels 4cg .. 4cg + 3 of step ts)
  u32x4_t mr[NBV];
  u32x2_t vr, zr = {0u, 0u};
  auto fetch = [&](int64_t c) {
    const int64_t t0 = c * kQ;
    const uint32_t rows = (uint32_t)(L - t0 < kQ ? L - t0 : (int64_t)kQ);
    const __amdgpu_buffer_rsrc_t rsm =
        make_rsrc(static_cast<const uint16_t*>(mat_in) + (b * L + t0) * N, rows * N * 2u);
    const uint32_t om = (uint32_t)ts * N * 2u + (uint32_t)(NB * cg) * 2u;
#pragma unroll
    for (int j = 0; j < NBV; ++j)
      mr[j] = __builtin_bit_cast(u32x4_t,
                                 __builtin_amdgcn_raw_buffer_load_b128(rsm, om + 16u * j, 0, 0));
    const uint32_t rb = rows * (uint32_t)dim * 2u;
    const uint32_t ox = (uint32_t)ts * (uint32_t)dim * 2u + (uint32_t)(cb + 4 * cg) * 2u;
    vr = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                     make_rsrc(static_cast<const uint16_t*>(fwd ? a.x : a.dy) + (b * L + t0) * dim,
                               rb),
                     ox, 0, 0));
    if (HAS_Z && !fwd)
      zr = __builtin_bit_cast(
          u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                       make_rsrc(static_cast<const uint16_t*>(a.z) + (b * L + t0) * dim, rb), ox,
                       0, 0));
  };

  fetch(fwd ? 0 : K - 1);
  for (int i = 0; i < K; ++i) {
    const int64_t c = fwd ? i : K - 1 - i;
    const int64_t t0 = c * kQ;
    const int rows = (int)(L - t0 < kQ ? L - t0 : kQ);
    // the state entering chunk c (forward) or the adjoint leaving it
    float* dst = out + (((size_t)b * K + c) * dim + d) * N + soff;
#pragma unroll
    for (int j = 0; j < NT2; ++j) *reinterpret_cast<f32x4_t*>(dst + 16 * j) = acc[j];

    __syncthreads();  // every read of the previous chunk's LDS is done
#pragma unroll
    for (int j = 0; j < NBV; ++j) *reinterpret_cast<u32x4_t*>(&sm.ms[ts][NB * cg + 8 * j]) = mr[j];
    float v[4];  // x, or dpre = dy SiLU(z)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float v0 = bf16_lo(vr[m]), v1 = bf16_hi(vr[m]);
      const bool gate = HAS_Z && !fwd;
      v[2 * m] = gate ? v0 * silu(bf16_lo(zr[m])) : v0;
      v[2 * m + 1] = gate ? v1 * silu(bf16_hi(zr[m])) : v1;
    }
    if (w == 3)
      chunk_steps(a.dt, b, L, t0, rows, H, h, Ah, EULER || Ah == 0.0f, lane, sm.s2, sm.coef,
                  sm.ein, sm.eout);
    __syncthreads();
    if (i + 1 < K) fetch(fwd ? c + 1 : c - 1);
    {
      // weight of step ts: exp(s_last - s_t) coef_t forward, exp(s_t) backward
      const float e = fwd ? sm.eout[ts] * sm.coef[ts] : sm.ein[ts];
      uint32_t hw0, lw0, hw1, lw1;
      split_bf16(e * v[0], e * v[1], hw0, lw0);
      split_bf16(e * v[2], e * v[3], hw1, lw1);
      *reinterpret_cast<u32x2_t*>(&sm.eh[ts][4 * cg]) = u32x2_t{hw0, hw1};
      *reinterpret_cast<u32x2_t*>(&sm.el[ts][4 * cg]) = u32x2_t{lw0, lw1};
    }
    __syncthreads();
    // acc[n][p] <- exp(s_last) acc + sum_t M[t][n] (weighted v)[t][p]: A
    // operand row n, slots t; B operand column p, slots t
    const float dec = fast_exp2(sm.s2[kQ - 1]);
    const int p = 16 * pt + r16;
    const u32x4_t eh = lds_col8(&sm.eh[8 * g][p], kRowX);
    const u32x4_t el = lds_col8(&sm.el[8 * g][p], kRowX);
#pragma unroll
    for (int j = 0; j < NT2; ++j) {
      const u32x4_t ma = lds_col8(&sm.ms[8 * g][16 * (nh * NT2 + j) + r16], N + 8);
      acc[j] *= dec;
      acc[j] = mfma_k32(ma, eh, acc[j]);
      acc[j] = mfma_k32(ma, el, acc[j]);
    }
  }
  if (!fwd) {
    float* d0 = a.dh0 + ((size_t)b * dim + d) * N + soff;
#pragma unroll
    for (int j = 0; j < NT2; ++j) *reinterpret_cast<f32x4_t*>(d0 + 16 * j) = acc[j];
  }
}

// dcoef/dA of the hold: dt^2 psi(u), u = dt A, psi(u) = (u e^u - e^u + 1)/u^2
// = sum_m (m-1) u^(m-2)/m!; the series to u^5 for |u| < 1/4, else the closed
// form (dt a - coef) / A.
__device__ __forceinline__ float hold_dcoef_da(float dtv, float Av, float av, float cf) {
  const float u = dtv * Av;
  if (__builtin_fabsf(u) < 0.25f) {
    float s = __builtin_fmaf(u, 1.0f / 5760.0f, 1.0f / 840.0f);
    s = __builtin_fmaf(u, s, 1.0f / 144.0f);
    s = __builtin_fmaf(u, s, 1.0f / 30.0f);
    s = __builtin_fmaf(u, s, 1.0f / 8.0f);
    s = __builtin_fmaf(u, s, 1.0f / 3.0f);
    s = __builtin_fmaf(u, s, 0.5f);
    return dtv * dtv * s;
  }
  return __builtin_fmaf(dtv, av, -cf) / Av;
}

// ---------------------------------------------------------------------------
// pass C: gradients of one chunk for a group of heads
// ---------------------------------------------------------------------------
template <int N>
struct ChunkSmem {
  alignas(16) uint16_t cs[kQ][N + 8];   // C, [t][n]
  alignas(16) uint16_t bs[kQ][N + 8];   // B, [t][n]
  alignas(16) uint16_t xs[kQ][kRowP];   // x of the head, [t][p]
  alignas(16) uint16_t dys[kQ][kRowP];  // dy
  alignas(16) uint16_t zs[kQ][kRowP];   // z
  alignas(16) uint16_t dph[kQ][kRowP];  // dpre, high part
  alignas(16) uint16_t dpl[kQ][kRowP];  // low part
  // masked matrices [i][j], high and low parts: 0 = E o M o coef_j,
  // 1 = E o M, 2 = E o G, 3 = E o G o coef_j (the block j > i stays zero)
  alignas(16) uint16_t mat[4][2][kQ][kRowT];
  alignas(16) float s2[kQ], coef[kQ], ein[kQ], eout[kQ], dtv[kQ];
  // per wave and step, sums over the wave's channels: u.x, dpre.(C h_in),
  // x.(B g_out)
  alignas(16) float red[4][kQ][3];
  alignas(16) float rowp[3][16], colp[3][16];  // row / column sums of R per tile
  alignas(16) float gam[4];                      // <g_out, h_in> per wave
};

// 8 waves: 0..3 own 16 channels each (ys, u, dx, dz, per-step sums), 4..7 a
// quarter of the states each (dB, dC, accumulated over the group's heads).
constexpr int kChunkThreads = 512;

template <int N, bool HAS_Z, bool EULER>
__global__ __launch_bounds__(kChunkThreads) void ssd_bwd_chunk_kernel(SsdBwdArgs a) {
  constexpr int NB = N / 8, NBV = NB / 8;
  constexpr int NTW = N / 64;  // 16-state tiles of dB, dC per wave
  extern __shared__ __align__(16) unsigned char ssd_bwd_smem_raw[];
  ChunkSmem<N>& sm = *reinterpret_cast<ChunkSmem<N>*>(ssd_bwd_smem_raw);
  const int grp = blockIdx.x, c = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int H = a.nheads, dim = a.dim, K = a.nchunks;
  const int64_t L = a.seqlen, t0 = (int64_t)c * kQ;
  const int rows = (int)(L - t0 < kQ ? L - t0 : kQ);
  const int h_begin = grp * kSsdBwdHeadsPerBlock;
  const int h_end = h_begin + kSsdBwdHeadsPerBlock < H ? h_begin + kSsdBwdHeadsPerBlock : H;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int ts = tid & (kQ - 1), cg = tid >> 5;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  // the (0, 1) block of every matrix is never written: zero it once
  for (int k = tid; k < 4 * 2 * 16 * 8; k += kChunkThreads) {
    const int m = k >> 7, r = (k >> 3) & 15, cc = k & 7;
    *reinterpret_cast<uint32_t*>(&sm.mat[m >> 1][m & 1][r][16 + 2 * cc]) = 0u;
  }
  // B and C of the chunk (shared by the group's heads), threads < 256
  if (tid < kThreads) {
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(
        static_cast<const uint16_t*>(a.B) + (b * L + t0) * N, (uint32_t)rows * N * 2u);
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(
        static_cast<const uint16_t*>(a.C) + (b * L + t0) * N, (uint32_t)rows * N * 2u);
    const uint32_t ob = (uint32_t)ts * N * 2u + (uint32_t)(NB * cg) * 2u;
#pragma unroll
    for (int j = 0; j < NBV; ++j) {
      *reinterpret_cast<u32x4_t*>(&sm.bs[ts][NB * cg + 8 * j]) = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsb, ob + 16u * j, 0, 0));
      *reinterpret_cast<u32x4_t*>(&sm.cs[ts][NB * cg + 8 * j]) = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsc, ob + 16u * j, 0, 0));
    }
  }
  __syncthreads();

  // waves 0..2 own the lower tiles (I, J) = (0,0), (1,0), (1,1) of the 32 x 32
  // matrices; lane value q is entry i = 16 I + r16, j = 16 J + 4 g + q
  const int I = w > 0 ? 1 : 0, J = w == 1 ? 0 : I;
  f32x4_t mt = zero4;  // (C B^T)[i][j], the same for every head
  if (w < 3) {
#pragma unroll
    for (int k = 0; k < N / 32; ++k)
      mt = mfma_k32(lds128(&sm.bs[16 * J + r16][32 * k + 8 * g]),
                    lds128(&sm.cs[16 * I + r16][32 * k + 8 * g]), mt);
  }

  // dB, dC of this wave's state tiles, summed over the group's heads:
  // [row tile][tile] in result layout (column n, rows t)
  f32x4_t accb[2][NTW], accc[2][NTW];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int k = 0; k < NTW; ++k) accb[r][k] = accc[r][k] = zero4;

  const uint32_t rb = (uint32_t)rows * (uint32_t)dim * 2u;
  const __amdgpu_buffer_rsrc_t rsx =
      make_rsrc(static_cast<const uint16_t*>(a.x) + (b * L + t0) * dim, rb);
  const __amdgpu_buffer_rsrc_t rsdy =
      make_rsrc(static_cast<const uint16_t*>(a.dy) + (b * L + t0) * dim, rb);
  const __amdgpu_buffer_rsrc_t rsz =
      make_rsrc(static_cast<const uint16_t*>(HAS_Z ? a.z : a.x) + (b * L + t0) * dim, rb);
  const __amdgpu_buffer_rsrc_t rsdx =
      make_rsrc(static_cast<uint16_t*>(a.dx) + (b * L + t0) * dim, rb);
  const __amdgpu_buffer_rsrc_t rsdz =
      make_rsrc(static_cast<uint16_t*>(HAS_Z ? a.dz : a.dx) + (b * L + t0) * dim, rb);

  // staging registers of waves 4..7: step ts, channels 8cg..8cg+7 of a head
  const int tsx = tid & (kQ - 1), cgx = (tid >> 5) & 7;
  u32x4_t xw = {0u, 0u, 0u, 0u}, dyw = xw, zw = xw;
  auto fetch_head = [&](int hh) {
    const uint32_t ox = (uint32_t)tsx * (uint32_t)dim * 2u + (uint32_t)(hh * kHD + 8 * cgx) * 2u;
    xw = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsx, ox, 0, 0));
    dyw = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsdy, ox, 0, 0));
    if constexpr (HAS_Z)
      zw = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsz, ox, 0, 0));
  };
  if (w >= 4) fetch_head(h_begin);
  uint32_t dt_raw = w == 3 ? load_dt(a.dt, b, L, t0, rows, H, h_begin, lane) : 0u;

  for (int h = h_begin; h < h_end; ++h) {
    const float Ah = a.A[h];
    __syncthreads();  // every read of the previous head's staging is done
    // ---- stage x, dy, z and dpre = dy SiLU(z) of head h (waves 4..7, from
    // registers loaded during the previous head), then load head h + 1 ----
    if (w >= 4) {
      *reinterpret_cast<u32x4_t*>(&sm.xs[tsx][8 * cgx]) = xw;
      *reinterpret_cast<u32x4_t*>(&sm.dys[tsx][8 * cgx]) = dyw;
      *reinterpret_cast<u32x4_t*>(&sm.zs[tsx][8 * cgx]) = zw;
      float dp[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float d0 = bf16_lo(dyw[m]), d1 = bf16_hi(dyw[m]);
        dp[2 * m] = HAS_Z ? d0 * silu(bf16_lo(zw[m])) : d0;
        dp[2 * m + 1] = HAS_Z ? d1 * silu(bf16_hi(zw[m])) : d1;
      }
      u32x4_t hi, lo;
      split8(dp, hi, lo);
      *reinterpret_cast<u32x4_t*>(&sm.dph[tsx][8 * cgx]) = hi;
      *reinterpret_cast<u32x4_t*>(&sm.dpl[tsx][8 * cgx]) = lo;
      if (h + 1 < h_end) fetch_head(h + 1);
    }
    if (w == 3) {
      chunk_steps_raw(dt_raw, Ah, EULER || Ah == 0.0f, lane, sm.s2, sm.coef, sm.ein, sm.eout,
                      sm.dtv);
      if (h + 1 < h_end) dt_raw = load_dt(a.dt, b, L, t0, rows, H, h + 1, lane);
    }
    __syncthreads();

    // ---- G = dpre x^T and the masked matrices (waves 0..2) -------------
    if (w < 3) {
      f32x4_t gt = zero4;  // G[i][j] = dpre_i . x_j, contraction over the 64 channels
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const u32x4_t xa = lds128(&sm.xs[16 * J + r16][32 * k + 8 * g]);
        gt = mfma_k32(xa, lds128(&sm.dph[16 * I + r16][32 * k + 8 * g]), gt);
        gt = mfma_k32(xa, lds128(&sm.dpl[16 * I + r16][32 * k + 8 * g]), gt);
      }
      const int i = 16 * I + r16;
      const float si = sm.s2[i];
      float v[4][4];  // [matrix][q]
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = 16 * J + 4 * g + q;
        const float e = j <= i ? fast_exp2(si - sm.s2[j]) : 0.0f;
        const float cj = sm.coef[j];
        v[1][q] = mt[q] * e;
        v[0][q] = v[1][q] * cj;
        v[2][q] = gt[q] * e;
        v[3][q] = v[2][q] * cj;
      }
      // R = P o G: row sums (over this lane's j, then the lane groups) and
      // column sums (over the 16 rows of the tile)
      float rr = 0.0f, cs4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cs4[q] = v[0][q] * gt[q];
        rr += cs4[q];
      }
      rr += __shfl_xor(rr, 16);
      rr += __shfl_xor(rr, 32);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) cs4[q] += __shfl_xor(cs4[q], o);
      if (g == 0) sm.rowp[w][r16] = rr;
      if (r16 == 0)
#pragma unroll
        for (int q = 0; q < 4; ++q) sm.colp[w][4 * g + q] = cs4[q];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t h0w, l0w, h1w, l1w;
        split_bf16(v[m][0], v[m][1], h0w, l0w);
        split_bf16(v[m][2], v[m][3], h1w, l1w);
        *reinterpret_cast<u32x2_t*>(&sm.mat[m][0][i][16 * J + 4 * g]) = u32x2_t{h0w, h1w};
        *reinterpret_cast<u32x2_t*>(&sm.mat[m][1][i][16 * J + 4 * g]) = u32x2_t{l0w, l1w};
      }
    }
    __syncthreads();

    const size_t sbase = (((size_t)b * K + c) * dim + h * kHD) * N;
    const float* hin = a.hbuf + sbase;
    const float* gout = a.gbuf + sbase;

    if (w < 4) {
    // ---- ys and u for channels p = 16 w + r16 (result column p, rows t) --
    const int p = 16 * w + r16;
    f32x4_t ys[2] = {zero4, zero4}, us[2] = {zero4, zero4};
    float gam = 0.0f;  // <g_out, h_in> over this lane's (channel, states)
    // two state steps at a time: the loads of all N/32 in flight together
    // would exceed the register budget of 8 waves
#pragma unroll 2
    for (int k = 0; k < N / 32; ++k) {
      // the states of channel p, states 32k + 8g .. + 7, as B operands
      const f32x4_t h0v = *reinterpret_cast<const f32x4_t*>(hin + p * N + 32 * k + 8 * g);
      const f32x4_t h1v = *reinterpret_cast<const f32x4_t*>(hin + p * N + 32 * k + 8 * g + 4);
      const f32x4_t g0v = *reinterpret_cast<const f32x4_t*>(gout + p * N + 32 * k + 8 * g);
      const f32x4_t g1v = *reinterpret_cast<const f32x4_t*>(gout + p * N + 32 * k + 8 * g + 4);
      const float hv[8] = {h0v[0], h0v[1], h0v[2], h0v[3], h1v[0], h1v[1], h1v[2], h1v[3]};
      const float gv[8] = {g0v[0], g0v[1], g0v[2], g0v[3], g1v[0], g1v[1], g1v[2], g1v[3]};
      u32x4_t hh, hl, gh, gl;
      split8(hv, hh, hl);
      split8(gv, gh, gl);
#pragma unroll
      for (int s = 0; s < 8; ++s) gam = __builtin_fmaf(gv[s], hv[s], gam);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const u32x4_t ca = lds128(&sm.cs[16 * r + r16][32 * k + 8 * g]);
        ys[r] = mfma_k32(ca, hh, ys[r]);
        ys[r] = mfma_k32(ca, hl, ys[r]);
        const u32x4_t ba = lds128(&sm.bs[16 * r + r16][32 * k + 8 * g]);
        us[r] = mfma_k32(ba, gh, us[r]);
        us[r] = mfma_k32(ba, gl, us[r]);
      }
    }
    // this lane's x and dpre (steps 16 r + 4 g + q, channel p)
    float xv[2][4], dpv[2][4], sa[2][4], sb[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = 16 * r + 4 * g + q;
        xv[r][q] = bf16_at(&sm.xs[t][p]);
        dpv[r][q] = bf16_at(&sm.dph[t][p]) + bf16_at(&sm.dpl[t][p]);
        sa[r][q] = dpv[r][q] * ys[r][q];  // dpre . (h_in^T C), this channel
        sb[r][q] = xv[r][q] * us[r][q];   // x . (g_out^T B)
      }
    {
      const u32x4_t xcol = lds_col8(&sm.xs[8 * g][p], kRowP);
      const u32x4_t dch = lds_col8(&sm.dph[8 * g][p], kRowP);
      const u32x4_t dcl = lds_col8(&sm.dpl[8 * g][p], kRowP);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ys[r][q] *= sm.ein[16 * r + 4 * g + q];
          us[r][q] *= sm.eout[16 * r + 4 * g + q];
        }
        // ys rows i = 16 r + r16 of matrix 0, slots j; x column p, slots j
        ys[r] = mfma_k32(lds128(&sm.mat[0][0][16 * r + r16][8 * g]), xcol, ys[r]);
        ys[r] = mfma_k32(lds128(&sm.mat[0][1][16 * r + r16][8 * g]), xcol, ys[r]);
        // u rows j = 16 r + r16 of matrix 1 transposed, slots i; dpre column p
        const u32x4_t lh = lds_col8(&sm.mat[1][0][8 * g][16 * r + r16], kRowT);
        const u32x4_t ll = lds_col8(&sm.mat[1][1][8 * g][16 * r + r16], kRowT);
        us[r] = mfma_k32(lh, dch, us[r]);
        us[r] = mfma_k32(lh, dcl, us[r]);
        us[r] = mfma_k32(ll, dch, us[r]);
      }
    }

    // ---- epilogue: dx, dz, D's partial sums, per-step sums --------------
    {
      const float Dp = a.Dskip ? a.Dskip[h * kHD + p] : 0.0f;
      float dd = 0.0f;
      float su[2][4];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = 16 * r + 4 * g + q;
          const float dyv = bf16_at(&sm.dys[t][p]);
          const float dxv = __builtin_fmaf(sm.coef[t], us[r][q], Dp * dpv[r][q]);
          const uint32_t off = (uint32_t)t * (uint32_t)dim * 2u + (uint32_t)(h * kHD + p) * 2u;
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(dxv), rsdx, off, 0, 0);
          if constexpr (HAS_Z) {
            const float zv = bf16_at(&sm.zs[t][p]);
            const float sg = sigmoid_f(zv);
            const float pre = __builtin_fmaf(Dp, xv[r][q], ys[r][q]);
            const float dzv = dyv * pre * sg * __builtin_fmaf(zv, 1.0f - sg, 1.0f);
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(dzv), rsdz, off, 0, 0);
          }
          dd = __builtin_fmaf(dpv[r][q], xv[r][q], dd);
          su[r][q] = us[r][q] * xv[r][q];
        }
      }
      // D: sum over the 32 steps of this channel (the four lane groups)
      dd += __shfl_xor(dd, 16);
      dd += __shfl_xor(dd, 32);
      if (g == 0 && a.dd_part)
        a.dd_part[((size_t)b * K + c) * dim + h * kHD + p] = dd;
      // per step: sums over the wave's 16 channels (lanes with the same g)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            su[r][q] += __shfl_xor(su[r][q], o);
            sa[r][q] += __shfl_xor(sa[r][q], o);
            sb[r][q] += __shfl_xor(sb[r][q], o);
          }
        }
      }
      if (r16 == 0) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float* rd = sm.red[w][16 * r + 4 * g + q];
            rd[0] = su[r][q];
            rd[1] = sa[r][q];
            rd[2] = sb[r][q];
          }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) gam += __shfl_xor(gam, o);
      if (lane == 0) sm.gam[w] = gam;
    }

    } else {
    // ---- dB and dC of this wave's state tiles ---------------------------
#pragma unroll
    for (int ti = 0; ti < NTW; ++ti) {
      const int n = 16 * (NTW * (w - 4) + ti) + r16;  // this lane's state (result column)
      f32x4_t tb[2] = {zero4, zero4}, tc[2] = {zero4, zero4};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
            // g_out and h_in of state n, channels 32k + 8g .. + 7, as B operands
        float gv[8], hv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          gv[s] = gout[(32 * k + 8 * g + s) * N + n];
          hv[s] = hin[(32 * k + 8 * g + s) * N + n];
        }
        u32x4_t gh, gl, hh, hl;
        split8(gv, gh, gl);
        split8(hv, hh, hl);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const u32x4_t xa = lds128(&sm.xs[16 * r + r16][32 * k + 8 * g]);
          tb[r] = mfma_k32(xa, gh, tb[r]);
          tb[r] = mfma_k32(xa, gl, tb[r]);
          const u32x4_t dah = lds128(&sm.dph[16 * r + r16][32 * k + 8 * g]);
          const u32x4_t dal = lds128(&sm.dpl[16 * r + r16][32 * k + 8 * g]);
          tc[r] = mfma_k32(dah, hh, tc[r]);
          tc[r] = mfma_k32(dah, hl, tc[r]);
          tc[r] = mfma_k32(dal, hh, tc[r]);
        }
      }
      const u32x4_t ccol = lds_col8(&sm.cs[8 * g][n], N + 8);
      const u32x4_t bcol = lds_col8(&sm.bs[8 * g][n], N + 8);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          tb[r][q] *= sm.eout[16 * r + 4 * g + q];
          tc[r][q] *= sm.ein[16 * r + 4 * g + q];
        }
        // dB rows j = 16 r + r16 of matrix 2 transposed (slots i), C column n
        const u32x4_t wh = lds_col8(&sm.mat[2][0][8 * g][16 * r + r16], kRowT);
        const u32x4_t wl = lds_col8(&sm.mat[2][1][8 * g][16 * r + r16], kRowT);
        tb[r] = mfma_k32(wh, ccol, tb[r]);
        tb[r] = mfma_k32(wl, ccol, tb[r]);
        // dC rows i = 16 r + r16 of matrix 3 (slots j), B column n
        tc[r] = mfma_k32(lds128(&sm.mat[3][0][16 * r + r16][8 * g]), bcol, tc[r]);
        tc[r] = mfma_k32(lds128(&sm.mat[3][1][16 * r + r16][8 * g]), bcol, tc[r]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          accb[r][ti][q] = __builtin_fmaf(sm.coef[16 * r + 4 * g + q], tb[r][q], accb[r][ti][q]);
          accc[r][ti][q] += tc[r][q];
        }
      }
    }
    }
    __syncthreads();  // per-step sums of all waves are in place
    if (w == 0) {
      // kappa of step t = lane (lanes < 32; the rest carry zeros)
      const int t = lane & (kQ - 1);
      const bool on = lane < kQ;
      float dc = 0.0f, al = 0.0f, be = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dc += sm.red[k][t][0];
        al += sm.red[k][t][1];
        be += sm.red[k][t][2];
      }
      const float row = t < 16 ? sm.rowp[0][t] : sm.rowp[1][t - 16] + sm.rowp[2][t - 16];
      const float col = t < 16 ? sm.colp[0][t] + sm.colp[1][t] : sm.colp[2][t - 16];
      const float cf = sm.coef[t], dtv = sm.dtv[t];
      al = on ? al * sm.ein[t] : 0.0f;             // alpha_t
      be = on ? be * sm.eout[t] * cf : 0.0f;       // beta_t
      float xr = on ? col - row + be : 0.0f;       // summed over steps < t
      // exclusive prefix of xr, inclusive suffix of al over the 32 lanes
      float pre = xr, suf = al;
#pragma unroll
      for (int o = 1; o < kQ; o <<= 1) {
        const float v = __shfl_up(pre, o);
        if (lane >= o) pre += v;
        const float u = __shfl_down(suf, o);
        if (lane + o < kQ) suf += u;
      }
      const float gamma = (sm.gam[0] + sm.gam[1] + sm.gam[2] + sm.gam[3]) *
                          fast_exp2(sm.s2[kQ - 1]);
      const float kappa = pre - xr + suf + gamma;
      const bool keep = on && t < rows;
      float da = 0.0f;
      if (keep) {
        const float av = fast_exp2(dtv * Ah * kLog2e);
        const float gd = __builtin_fmaf(kappa, Ah, EULER ? dc : dc * av);
        static_cast<uint16_t*>(a.ddt)[((size_t)b * L + t0 + t) * H + h] = f32_to_bf16_bits(gd);
        da = kappa * dtv;
        if (!EULER) da = __builtin_fmaf(dc, hold_dcoef_da(dtv, Ah, av, cf), da);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) da += __shfl_xor(da, o);
      if (lane == 0) a.da_part[((size_t)b * K + c) * H + h] = da;
    }
  }

  // dB, dC partial sums of the group
  if (w < 4) return;
  const int G = a.ngroups;
#pragma unroll
  for (int ti = 0; ti < NTW; ++ti) {
    const int n = 16 * (NTW * (w - 4) + ti) + r16;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = 16 * r + 4 * g + q;
        if (t < rows) {
          const size_t o = (((size_t)b * L + t0 + t) * G + grp) * N + n;
          a.db_part[o] = accb[r][ti][q];
          a.dc_part[o] = accc[r][ti][q];
        }
      }
  }
}

// ---------------------------------------------------------------------------
// pass D
// ---------------------------------------------------------------------------
// dB, dC: sums over the head groups, rounded to bf16
__global__ __launch_bounds__(256) void ssd_bwd_sum_groups_kernel(SsdBwdArgs a) {
  const int N = a.dstate, G = a.ngroups;
  const int64_t n_all = a.batch * a.seqlen * N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_all) return;
  const int64_t r = i / N;
  const int n = (int)(i % N);
  float sb = 0.0f, sc = 0.0f;
  for (int k = 0; k < G; ++k) {
    sb += a.db_part[(r * G + k) * N + n];
    sc += a.dc_part[(r * G + k) * N + n];
  }
  static_cast<uint16_t*>(a.dB)[i] = f32_to_bf16_bits(sb);
  static_cast<uint16_t*>(a.dC)[i] = f32_to_bf16_bits(sc);
}

// dD: sums over (batch row, chunk); a block takes 64 channels, its 4 waves
// every 4th row, combined in a fixed order
__global__ __launch_bounds__(256) void ssd_bwd_sum_dd_kernel(SsdBwdArgs a) {
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = blockIdx.x * 64 + lane;
  const int64_t rows = a.batch * a.nchunks;
  float s = 0.0f;
  if (d < a.dim) {
#pragma unroll 8
    for (int64_t r = w; r < rows; r += 4) s += a.dd_part[r * a.dim + d];
  }
  part[w][lane] = s;
  __syncthreads();
  if (w == 0 && d < a.dim) a.dD[d] = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
}

// dA: one wave per head, sums over (batch row, chunk)
__global__ __launch_bounds__(64) void ssd_bwd_sum_da_kernel(SsdBwdArgs a) {
  const int h = blockIdx.x, lane = threadIdx.x;
  const int64_t rows = a.batch * a.nchunks;
  float s = 0.0f;
#pragma unroll 4
  for (int64_t r = lane; r < rows; r += 64) s += a.da_part[r * a.nheads + h];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) a.dA[h] = s;
}

template <int N, bool HAS_Z, bool EULER>
hipError_t launch_chunk_passes(const SsdBwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((ssd_bwd_walk_kernel<N, HAS_Z, EULER>),
                     dim3(4 * a.nheads, (unsigned)a.batch), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto kern = ssd_bwd_chunk_kernel<N, HAS_Z, EULER>;
  const size_t smem = sizeof(ChunkSmem<N>);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.ngroups, a.nchunks, (unsigned)a.batch), dim3(kChunkThreads),
                     smem, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nbc = a.batch * a.seqlen * N;
  hipLaunchKernelGGL(ssd_bwd_sum_groups_kernel, dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0,
                     stream, a);
  hipLaunchKernelGGL(ssd_bwd_sum_da_kernel, dim3(a.nheads), dim3(64), 0, stream, a);
  if (a.dD)
    hipLaunchKernelGGL(ssd_bwd_sum_dd_kernel, dim3((a.dim + 63) / 64), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int N>
hipError_t launch_chunk_passes_n(const SsdBwdArgs& a, hipStream_t stream) {
  if (a.z) return a.euler ? launch_chunk_passes<N, true, true>(a, stream)
                          : launch_chunk_passes<N, true, false>(a, stream);
  return a.euler ? launch_chunk_passes<N, false, true>(a, stream)
                 : launch_chunk_passes<N, false, false>(a, stream);
}

}  // namespace

hipError_t launch_ssd_bwd_mm(const SsdBwdArgs& a, hipStream_t stream) {
  switch (a.dstate) {
    case 64: return launch_chunk_passes_n<64>(a, stream);
    case 128: return launch_chunk_passes_n<128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssm
