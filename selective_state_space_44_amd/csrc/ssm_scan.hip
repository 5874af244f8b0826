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
//   * B[b,t,n] and C[b,t,n] are the same for all 64 lanes of a wave.  B is
//     loaded into a few VGPRs, 16 (step, state) values per register repeated
//     in each 16-lane row, and handed to the multiply that needs it through a
//     DPP row broadcast fused into that instruction.  C is written to a small
//     per-wave LDS slice one tile ahead and read back with broadcast 16-byte
//     LDS loads.  x, delta and z are read once per lane per step (one
//     coalesced row segment per wave) through a buffer resource whose row
//     offset is a scalar, so the inner loop does no per-lane address
//     arithmetic.
//   * Software pipeline: the loads of tile i+1 are in flight while tile i is
//     computed (ping-pong register sets), and within a tile the exp2 and
//     input terms of step group j+1 are formed before the serial updates of
//     group j so that their latency hides behind the recurrence.
//   * Update form: with q = B*x/A, Bbar*x = (Abar - 1)*q = fma(Abar, q, -q)
//     and the state update is the single fma h = fma(Abar, h, Bbar*x), with
//     Abar = exp2(delta * A*log2(e)).  A zero step (Abar == 1, Bbar == 0)
//     leaves the state bit-for-bit unchanged.
//   * Readout: each wave forms its partial sum over its NPL states for every
//     step of a T-step tile (wave 0 also adds D*x), writes it to LDS, and
//     after one barrier wave g finishes steps s = g, g+G, ... of the tile:
//     sum of the G partials (fixed order, so results are deterministic),
//     SiLU gate, and one coalesced store of y.
//   * Sequence chunks (paperlens tutorial, parallel-scan section: the update
//     h_t = Abar_t h_{t-1} + u_t composes associatively): when the plan cuts
//     L into K chunks, a first kernel runs every chunk but the last from a
//     zero state and records its end state hloc_c and sum of delta; a carry
//     kernel composes the affine maps h -> P_c h + hloc_c with
//     P_c = exp(A * sum(delta over chunk c)) in chunk order; the main kernel
//     then runs every chunk from its true entering state.
//   * A == 0 (which the ZOH formula reaches only as a limit) switches the
//     affected wave to a form with that limit, Bbar = delta * B.

#include <type_traits>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

constexpr int kChunkAlign = 16;  // chunks start on a multiple of this many steps

// One ZOH step of NPL states of one channel (unpipelined form).
template <int NPL, bool ZERO_A>
__device__ __forceinline__ void zoh_step(float dv, float xv, const float* Bv,
                                         const float (&A2)[NPL], const float (&iA)[NPL],
                                         float (&h)[NPL]);

// ZOH coefficients of one (step, state): h' = a*h + b with a = Abar and
// b = Bbar*x.  With q = B*x/A, Bbar*x = (Abar - 1)*q = fma(Abar, q, -q), so
// the recurrence itself is a single fma (h' = fma(a, h, b)) and a step of
// zero length (a == 1, b == 0) leaves the state bit-for-bit unchanged.
// Where A == 0 (iA is +-inf) the limit Bbar = delta*B is used instead.
template <bool ZERO_A>
__device__ __forceinline__ void zoh_coef(float ds, float bx, float A2, float iA, float& a,
                                         float& b) {
  a = fast_exp2(ds * A2);
  if constexpr (!ZERO_A) {
    const float q = bx * iA;
    b = __builtin_fmaf(a, q, -q);
  } else {
    const bool lim = __builtin_isinf(iA);
    b = (lim ? ds : (a - 1.0f) * iA) * bx;
  }
}

template <int NPL, bool ZERO_A>
__device__ __forceinline__ void zoh_step(float dv, float xv, const float* Bv,
                                         const float (&A2)[NPL], const float (&iA)[NPL],
                                         float (&h)[NPL]) {
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    float a, b;
    zoh_coef<ZERO_A>(dv, Bv[k] * xv, A2[k], iA[k], a, b);
    h[k] = __builtin_fmaf(a, h[k], b);
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

// Raw (undecoded) I/O element as loaded: bf16 bits in the low half, or fp32.
template <typename IO> struct Raw;
template <> struct Raw<float> {
  using T = float;
  __device__ __forceinline__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
    return buf<float>::load(r, v, s);
  }
  __device__ __forceinline__ static float f(T v) { return v; }
};
template <> struct Raw<bf16> {
  using T = uint32_t;
  __device__ __forceinline__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, v, s, 0);
  }
  __device__ __forceinline__ static float f(T v) { return bf16_bits_to_f32(v); }
};

// Value of lane K of this lane's 16-lane row (DPP row_newbcast).  Written
// as a DPP move; the compiler folds it into the consuming VOP2 instruction,
// so the broadcast costs no extra instruction.
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + K, 0xf, 0xf, true));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time loop).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
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

// How one wave holds the B and C values of its NPL states for a tile of
// T steps (T*NPL values each):
//  * B lives in NPL VGPRs, 16 values per register, the same 16 in each of the
//    four 16-lane rows: value v = step*NPL + k sits in register v/16, lane
//    v%16 of every row, and is read with row_bcast<v%16>;
//  * C is staged in LDS (16*NPL floats per tile, double buffered, per wave)
//    and read with one broadcast LDS load per step.
template <int NPL, int T>
struct BCLayout {
  static constexpr int kVals = T * NPL;                           // B (or C) values per tile
  static constexpr int kBRegs = (kVals + 15) / 16;                // B VGPRs per tile
  static constexpr int kCVals = kVals;                            // C floats per tile
  static constexpr int kCPerLane = (kVals + kWave - 1) / kWave;   // C values loaded per lane
};

template <typename IO, int NPL, int T>
struct BCRegs {
  typename Raw<IO>::T b[BCLayout<NPL, T>::kBRegs], c[BCLayout<NPL, T>::kCPerLane];
};

// Per-lane byte offsets (within a tile's rows of B or C) of the values this
// lane loads.
template <typename IO, int NPL, int T>
struct BCOffsets {
  using L = BCLayout<NPL, T>;
  uint32_t b[L::kBRegs], c[L::kCPerLane];
  int cslot[L::kCPerLane];  // LDS slot of each C value
  __device__ __forceinline__ BCOffsets(int lane, int n0) {
    const int p = lane % 16;
#pragma unroll
    for (int r = 0; r < L::kBRegs; ++r) {
      const int v = min(16 * r + p, L::kVals - 1);
      b[r] = (uint32_t)(((v / NPL) * kDState + n0 + v % NPL) * sizeof(IO));
    }
#pragma unroll
    for (int r = 0; r < L::kCPerLane; ++r) {
      const int v = (lane + kWave * r) % L::kCVals;
      cslot[r] = v;
      c[r] = (uint32_t)(((v / NPL) * kDState + n0 + v % NPL) * sizeof(IO));
    }
  }
};

// Rows of one chunk of a [b, L, 16] tensor (B or C) as a buffer.
template <typename IO>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bc_rsrc(const IO* p, const Chunk& k,
                                                          int64_t seqlen) {
  const size_t first = ((size_t)k.b * seqlen + k.t_begin) * kDState;
  return make_rsrc(p + first, (uint32_t)((size_t)(k.t_end - k.t_begin) * kDState * sizeof(IO)));
}

// ---------------------------------------------------------------------------
// Main scan: one chunk of 64 channels x all 16 states per block.
// ---------------------------------------------------------------------------
template <typename IO, int G, int T>
struct TileRegs {
  typename Raw<IO>::T x[T], d[T], z[(T + G - 1) / G];
  BCRegs<IO, kDState / G, T> bc;
};

template <int NPL>
__device__ __forceinline__ void read_c(const float* cst, int s, float (&cv)[NPL]) {
  if constexpr (NPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(cst + s * NPL)[q];
      cv[4 * q] = v.x;
      cv[4 * q + 1] = v.y;
      cv[4 * q + 2] = v.z;
      cv[4 * q + 3] = v.w;
    }
  } else if constexpr (NPL == 2) {
    const float2 v = reinterpret_cast<const float2*>(cst + s * NPL)[0];
    cv[0] = v.x;
    cv[1] = v.y;
  } else {
    cv[0] = cst[s];
  }
}

template <typename IO, int G, int T, bool HAS_Z, bool ZERO_A>
__device__ __forceinline__ void scan_chunk(const IO* __restrict__ x, const IO* __restrict__ delta,
                                           const IO* __restrict__ B, const IO* __restrict__ C,
                                           const IO* __restrict__ z, IO* __restrict__ y,
                                           float Dd, int64_t seqlen, int dim, const Chunk& k,
                                           float* part, float* cst,
                                           const float (&A2)[kDState / G],
                                           const float (&iA)[kDState / G],
                                           float (&h)[kDState / G]) {
  constexpr int NPL = kDState / G;
  constexpr int ZT = (T + G - 1) / G;  // steps of a tile this wave finishes (at most)
  constexpr int SG = NPL >= 8 ? 1 : 8 / NPL;  // steps per coefficient group
  static_assert(T % SG == 0, "tile must split into groups");
  using R = Raw<IO>;
  using L = BCLayout<NPL, T>;
  const __amdgpu_buffer_rsrc_t rx = rows_rsrc(x, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t rd = rows_rsrc(delta, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t rz = rows_rsrc(HAS_Z ? z : x, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t ry = rows_rsrc(y, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t rb = bc_rsrc(B, k, seqlen);
  const __amdgpu_buffer_rsrc_t rc = bc_rsrc(C, k, seqlen);
  const BCOffsets<IO, NPL, T> bco(k.lane, k.g * NPL);
  const uint32_t voff = (uint32_t)k.d * sizeof(IO);
  // lanes past the last channel store out of the buffer's range (dropped)
  const uint32_t voff_y = k.active ? voff : 0x80000000u;
  const uint32_t row_bytes = (uint32_t)dim * sizeof(IO);
  const int nsteps = (int)(k.t_end - k.t_begin);
  const int nfull = nsteps / T;
  const float dmul = (k.g == 0) ? Dd : 0.0f;  // wave 0 carries the skip term

  // Loads of tile `tidx` into r.  Prefetches past the last full tile are
  // clamped onto it (their values are never used).
  auto issue = [&](TileRegs<IO, G, T>& r, int tidx) {
    const int s0 = min(tidx, nfull - 1) * T;
    const uint32_t bcs = (uint32_t)s0 * kDState * sizeof(IO);
#pragma unroll
    for (int j = 0; j < L::kCPerLane; ++j) r.bc.c[j] = R::load(rc, bco.c[j], bcs);
#pragma unroll
    for (int j = 0; j < L::kBRegs; ++j) r.bc.b[j] = R::load(rb, bco.b[j], bcs);
#pragma unroll
    for (int s = 0; s < T; ++s) {
      const uint32_t so = (uint32_t)(s0 + s) * row_bytes;
      r.x[s] = R::load(rx, voff, so);
      r.d[s] = R::load(rd, voff, so);
    }
    if constexpr (HAS_Z) {
#pragma unroll
      for (int j = 0; j < ZT; ++j)
        r.z[j] = R::load(rz, voff, (uint32_t)min(s0 + k.g + j * G, nsteps - 1) * row_bytes);
    }
  };
  auto stage_c = [&](const TileRegs<IO, G, T>& r, int cb) {
#pragma unroll
    for (int j = 0; j < L::kCPerLane; ++j) cst[cb * L::kCVals + bco.cslot[j]] = R::f(r.bc.c[j]);
  };

  int pbuf = 0;
  auto tile = [&](const TileRegs<IO, G, T>& r, int tidx, int cb, const TileRegs<IO, G, T>& next,
                  bool has_next) {
    const int s0 = tidx * T;
    float bf[L::kBRegs];
#pragma unroll
    for (int j = 0; j < L::kBRegs; ++j) bf[j] = R::f(r.bc.b[j]);
    const float* cs = cst + cb * L::kCVals;
    // Coefficients (exp2 and the input term) of step group j+1 are formed
    // before the serial updates of group j, so the exp latency and the
    // coefficient math overlap the recurrence.
    float* pw = part + pbuf * (G * T * kWave) + k.g * T * kWave + k.lane;  // this wave's partials
    float ca[2][SG][NPL], cb2[2][SG][NPL], cc[2][SG][NPL];
    auto coefs = [&](auto gc, float (&a)[SG][NPL], float (&bb)[SG][NPL], float (&c)[SG][NPL]) {
      constexpr int g0 = decltype(gc)::value * SG;
      static_for<SG>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int s = g0 + i;
        read_c<NPL>(cs, s, c[i]);
        const float xs = R::f(r.x[s]);
        const float ds = R::f(r.d[s]);
        static_for<NPL>([&](auto nc) {
          constexpr int n = decltype(nc)::value;
          constexpr int v = s * NPL + n;  // B value (step, state) in the tile
          zoh_coef<ZERO_A>(ds, row_bcast<v % 16>(bf[v / 16]) * xs, A2[n], iA[n], a[i][n],
                           bb[i][n]);
        });
      });
    };
    coefs(std::integral_constant<int, 0>{}, ca[0], cb2[0], cc[0]);
    static_for<T / SG>([&](auto gc) {
      constexpr int gi = decltype(gc)::value;
      if constexpr (gi + 1 < T / SG)
        coefs(std::integral_constant<int, gi + 1>{}, ca[(gi + 1) & 1], cb2[(gi + 1) & 1],
              cc[(gi + 1) & 1]);
      // keep the next group's loads and exp2s ahead of this group's updates
      // (the scheduler would otherwise sink them next to their uses)
      __builtin_amdgcn_sched_barrier(0);
      static_for<SG>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int s = gi * SG + i;
        float acc = dmul * R::f(r.x[s]);
        static_for<NPL>([&](auto nc) {
          constexpr int n = decltype(nc)::value;
          h[n] = __builtin_fmaf(ca[gi & 1][i][n], h[n], cb2[gi & 1][i][n]);
          acc = __builtin_fmaf(cc[gi & 1][i][n], h[n], acc);
        });
        if constexpr (G == 1) {
          const float yv = HAS_Z ? acc * silu(R::f(r.z[s])) : acc;
          buf<IO>::store(yv, ry, voff_y, (uint32_t)(s0 + s) * row_bytes);
        } else {
          pw[s * kWave] = acc;
        }
      });
    });
    if (has_next) stage_c(next, cb ^ 1);
    if constexpr (G > 1) {
      float* pb = part + pbuf * (G * T * kWave);
      __syncthreads();
      // all partial sums first (one batch of LDS reads), then the epilogue
      float ps[ZT][G];
#pragma unroll
      for (int j = 0; j < ZT; ++j) {
        const int s = min(k.g + j * G, T - 1);
#pragma unroll
        for (int w = 0; w < G; ++w) ps[j][w] = pb[(w * T + s) * kWave + k.lane];
      }
#pragma unroll
      for (int j = 0; j < ZT; ++j) {
        const int s = k.g + j * G;
        if (T % G != 0 && s >= T) break;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < G; ++w) sum += ps[j][w];
        const float yv = HAS_Z ? sum * silu(R::f(r.z[j])) : sum;
        buf<IO>::store(yv, ry, voff_y, (uint32_t)(s0 + s) * row_bytes);
      }
      pbuf ^= 1;
    }
  };

  // full tiles, two at a time through the ping-pong register sets
  TileRegs<IO, G, T> ra, rb2;
  if (nfull > 0) {
    issue(ra, 0);
    stage_c(ra, 0);
  }
  int i = 0;
  for (; i + 2 <= nfull; i += 2) {
    issue(rb2, i + 1);
    tile(ra, i, 0, rb2, true);
    issue(ra, i + 2);
    tile(rb2, i + 1, 1, ra, true);
  }
  if (i < nfull) tile(ra, i, 0, ra, false);

  // ragged end of the chunk: one step at a time, no pipelining
  for (int s0 = nfull * T; s0 < nsteps; ++s0) {
    const uint32_t so = (uint32_t)s0 * row_bytes;
    const float xs = buf<IO>::load(rx, voff, so);
    const float ds = buf<IO>::load(rd, voff, so);
    const uint32_t bo = (uint32_t)(s0 * kDState + k.g * NPL) * sizeof(IO);
    float acc = dmul * xs;
#pragma unroll
    for (int n = 0; n < NPL; ++n) {
      const float Bn = buf<IO>::load(rb, bo + n * sizeof(IO), 0);
      const float Cn = buf<IO>::load(rc, bo + n * sizeof(IO), 0);
      float a, b;
      zoh_coef<ZERO_A>(ds, Bn * xs, A2[n], iA[n], a, b);
      h[n] = __builtin_fmaf(a, h[n], b);
      acc = __builtin_fmaf(Cn, h[n], acc);
    }
    if constexpr (G == 1) {
      const float yv = HAS_Z ? acc * silu(buf<IO>::load(rz, voff, so)) : acc;
      buf<IO>::store(yv, ry, voff_y, so);
    } else {
      float* pb = part + pbuf * (G * T * kWave);
      pb[(k.g * T) * kWave + k.lane] = acc;
      __syncthreads();
      if (k.g == 0) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < G; ++w) sum += pb[(w * T) * kWave + k.lane];
        const float yv = HAS_Z ? sum * silu(buf<IO>::load(rz, voff, so)) : sum;
        buf<IO>::store(yv, ry, voff_y, so);
      }
      pbuf ^= 1;
    }
  }
}
template <typename IO, int G, int T, bool HAS_Z>
__global__ __launch_bounds__(kWave* G) void scan_fwd_kernel(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, const IO* __restrict__ C, const float* __restrict__ Dskip,
    const IO* __restrict__ z, const float* __restrict__ h0, IO* __restrict__ y,
    float* __restrict__ h_last, const float* __restrict__ ws_hin, int64_t seqlen,
    int64_t chunk_len, int dim, int nchunks) {
  constexpr int NPL = kDState / G;
  __shared__ float part[G > 1 ? 2 * G * T * kWave : 1];
  __shared__ float cst_all[G * 2 * BCLayout<NPL, T>::kCVals];
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
  float* cst = cst_all + k.g * 2 * BCLayout<NPL, T>::kCVals;

  if (__builtin_amdgcn_ballot_w64(zero) != 0)
    scan_chunk<IO, G, T, HAS_Z, true>(x, delta, B, C, z, y, Dd, seqlen, dim, k, part, cst, A2,
                                      iA, h);
  else
    scan_chunk<IO, G, T, HAS_Z, false>(x, delta, B, C, z, y, Dd, seqlen, dim, k, part, cst, A2,
                                       iA, h);

  if (k.c == nchunks - 1 && h_last && k.active) {
    float* hl = h_last + ((size_t)k.b * dim + k.d) * kDState + n0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) hl[j] = h[j];
  }
}

// ---------------------------------------------------------------------------
// Carry pass 1: end state of every chunk but the last, started from zero,
// plus the chunk's sum of delta (accumulated in fp64).  Same pipelining and
// B layout as the main kernel, without the readout.
// ---------------------------------------------------------------------------
template <typename IO, int G, int T, bool ZERO_A>
__device__ __forceinline__ void chunk_state(const IO* __restrict__ x,
                                            const IO* __restrict__ delta,
                                            const IO* __restrict__ B, int64_t seqlen, int dim,
                                            const Chunk& k, const float (&A2)[kDState / G],
                                            const float (&iA)[kDState / G],
                                            float (&h)[kDState / G], double& sd) {
  constexpr int NPL = kDState / G;
  using R = Raw<IO>;
  using L = BCLayout<NPL, T>;
  const __amdgpu_buffer_rsrc_t rx = rows_rsrc(x, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t rd = rows_rsrc(delta, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t rb = bc_rsrc(B, k, seqlen);
  const BCOffsets<IO, NPL, T> bco(k.lane, k.g * NPL);
  const uint32_t voff = (uint32_t)k.d * sizeof(IO);
  const uint32_t row_bytes = (uint32_t)dim * sizeof(IO);
  const int nsteps = (int)(k.t_end - k.t_begin);
  const int nfull = nsteps / T;

  struct Regs {
    typename R::T x[T], d[T], b[L::kBRegs];
  };
  auto issue = [&](Regs& r, int tidx) {
    const int s0 = min(tidx, nfull - 1) * T;
    const uint32_t bcs = (uint32_t)s0 * kDState * sizeof(IO);
#pragma unroll
    for (int j = 0; j < L::kBRegs; ++j) r.b[j] = R::load(rb, bco.b[j], bcs);
#pragma unroll
    for (int s = 0; s < T; ++s) {
      const uint32_t so = (uint32_t)(s0 + s) * row_bytes;
      r.x[s] = R::load(rx, voff, so);
      r.d[s] = R::load(rd, voff, so);
    }
  };
  auto tile = [&](const Regs& r) {
    float bf[L::kBRegs];
#pragma unroll
    for (int j = 0; j < L::kBRegs; ++j) bf[j] = R::f(r.b[j]);
    static_for<T>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const float xs = R::f(r.x[s]);
      const float ds = R::f(r.d[s]);
      static_for<NPL>([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        constexpr int v = s * NPL + n;
        float a, b;
        zoh_coef<ZERO_A>(ds, row_bcast<v % 16>(bf[v / 16]) * xs, A2[n], iA[n], a, b);
        h[n] = __builtin_fmaf(a, h[n], b);
      });
      sd += (double)ds;
    });
  };
  Regs ra, rb2;
  if (nfull > 0) issue(ra, 0);
  int i = 0;
  for (; i + 2 <= nfull; i += 2) {
    issue(rb2, i + 1);
    tile(ra);
    issue(ra, i + 2);
    tile(rb2);
  }
  if (i < nfull) tile(ra);
  for (int s0 = nfull * T; s0 < nsteps; ++s0) {
    const uint32_t so = (uint32_t)s0 * row_bytes;
    const float xs = buf<IO>::load(rx, voff, so);
    const float ds = buf<IO>::load(rd, voff, so);
    const uint32_t bo = (uint32_t)(s0 * kDState + k.g * NPL) * sizeof(IO);
    float Bv[NPL];
#pragma unroll
    for (int n = 0; n < NPL; ++n) Bv[n] = buf<IO>::load(rb, bo + n * sizeof(IO), 0);
    zoh_step<NPL, ZERO_A>(ds, xs, Bv, A2, iA, h);
    sd += (double)ds;
  }
}

template <typename IO, int G, int T>
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
    chunk_state<IO, G, T, true>(x, delta, B, seqlen, dim, k, A2, iA, h, sd);
  else
    chunk_state<IO, G, T, false>(x, delta, B, seqlen, dim, k, A2, iA, h, sd);
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

template <typename IO, int G>
hipError_t launch_scan_t(const ScanArgs& a, int phase, hipStream_t stream) {
  constexpr int T = 8;  // steps per tile (chunks are whole multiples of it)
  const IO* x = static_cast<const IO*>(a.x);
  const IO* delta = static_cast<const IO*>(a.delta);
  const IO* B = static_cast<const IO*>(a.B);
  const IO* C = static_cast<const IO*>(a.C);
  const unsigned gx = (unsigned)((a.dim + kWave - 1) / kWave);
  if (a.nchunks > 1 && (phase & 1)) {
    dim3 grid1(gx, (unsigned)(a.nchunks - 1), (unsigned)a.batch);
    hipLaunchKernelGGL((scan_chunk_state_kernel<IO, G, T>), grid1, dim3(kWave * G), 0, stream, x,
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
  if (!(phase & 2)) return hipSuccess;
  dim3 grid(gx, (unsigned)a.nchunks, (unsigned)a.batch);
  if (a.z)
    hipLaunchKernelGGL((scan_fwd_kernel<IO, G, T, true>), grid, dim3(kWave * G), 0, stream, x,
                       delta, a.A, B, C, a.Dskip, static_cast<const IO*>(a.z), a.h0,
                       static_cast<IO*>(a.y), a.h_last, a.ws_hin, a.seqlen, a.chunk_len, a.dim,
                       a.nchunks);
  else
    hipLaunchKernelGGL((scan_fwd_kernel<IO, G, T, false>), grid, dim3(kWave * G), 0, stream, x,
                       delta, a.A, B, C, a.Dskip, static_cast<const IO*>(nullptr), a.h0,
                       static_cast<IO*>(a.y), a.h_last, a.ws_hin, a.seqlen, a.chunk_len, a.dim,
                       a.nchunks);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_scan_io(const ScanArgs& a, int G, int phase, hipStream_t stream) {
  switch (G) {
    case 2: return launch_scan_t<IO, 2>(a, phase, stream);
    case 4: return launch_scan_t<IO, 4>(a, phase, stream);
    case 8: return launch_scan_t<IO, 8>(a, phase, stream);
    case 16: return launch_scan_t<IO, 16>(a, phase, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int scan_tile_steps() { return kChunkAlign; }

ScanWorkspace scan_workspace_layout(int64_t batch, int64_t dim, int nchunks) {
  auto align = [](size_t v) { return (v + 255) & ~size_t(255); };
  ScanWorkspace w{0, 0, 0, 0};
  if (nchunks > 1) {
    const size_t states = (size_t)batch * nchunks * dim * kDState;
    w.hloc_off = 0;
    w.hin_off = w.hloc_off + align(states * sizeof(float));
    w.sdelta_off = w.hin_off + align(states * sizeof(float));
    w.total = w.sdelta_off + align((size_t)batch * nchunks * dim * sizeof(double));
  }
  return w;
}

hipError_t launch_scan(const ScanArgs& a, bool io_bf16, int waves_per_group, int phase,
                       hipStream_t stream) {
  return io_bf16 ? launch_scan_io<bf16>(a, waves_per_group, phase, stream)
                 : launch_scan_io<float>(a, waves_per_group, phase, stream);
}

hipError_t launch_copy_state(const float* h0, float* h_last, int64_t count,
                             hipStream_t stream) {
  hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     stream, h0, h_last, count);
  return hipGetLastError();
}

}  // namespace ssm
