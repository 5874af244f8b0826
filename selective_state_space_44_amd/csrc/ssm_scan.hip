// ssm_scan.hip -- selective scan forward kernels for gfx950 (wave64).
//
// Computes, per batch b, channel d, state n and step t (ultralytics glossary
// "State Space Models (SSM)", section "SSMの仕組み"; paperlens tutorial
// "Mamba と状態空間モデル", eq.(2) and the selection section):
//   Abar = exp(delta[b,t,d] * A[d,n]),  Bbar = (Abar - 1) / A[d,n] * B[b,t,n]
//   h    = Abar * h + Bbar * x[b,t,d]
//   y[b,t,d] = (sum_n C[b,t,n] h[n] + D[d] x[b,t,d]) * SiLU(z[b,t,d])
//
// Work decomposition (no MFMA: nothing here is a dense contraction; the
// kernels are bound by VALU issue, so the design minimises VALU cycles per
// element).
//   * A block owns 64 consecutive channels of one batch row and one chunk of
//     the sequence.  Lane j of every wave holds channel d0 + j; the block has
//     G waves and wave g holds the NPL = 16/G state indices
//     n in [g*NPL, (g+1)*NPL) of those 64 channels.  The fp32 state lives in
//     VGPRs for the whole chunk and never touches HBM.
//   * Inputs are staged per block through LDS in tiles of kT steps, two
//     stages deep: x and delta as fp32 rows [channel][step] (each wave reads
//     its lane's steps with 16-byte LDS loads), B and C as fp32 [step][state]
//     (read with broadcast LDS loads: every lane of a wave wants the same
//     values).  The fetch of a tile from HBM is shared evenly by the G
//     waves of the block and runs two tiles ahead of its use.  bf16 inputs
//     are widened for free: the 16 raw bits are written into the upper half of an fp32 LDS
//     slot whose lower half was zeroed once, so no VALU op converts them.
//   * Per element the main pass issues 6 fp32 VALU ops and one exp2:
//     a = exp2(delta * A*log2 e), q = (B*x) * (1/A), Bbar*x = fma(a, q, -q),
//     h = fma(a, h, Bbar*x), and one fma of the readout.  A zero step
//     (a == 1, Bbar*x == 0) leaves the state bit-for-bit unchanged.  The exp2
//     and input terms of step group j+1 are formed before the serial updates
//     of group j so that their latency hides behind the recurrence.
//   * Readout: each wave writes its partial sum over its NPL states for every
//     step of a tile to LDS; after the tile's one barrier, wave g finishes
//     steps s = g, g+G, ...: sum of the G partials in a fixed order (results
//     are deterministic), + D*x, SiLU gate, one coalesced store of y.
//   * Sequence chunks (paperlens tutorial, parallel-scan section: the update
//     h_t = Abar_t h_{t-1} + u_t composes associatively): when the plan cuts
//     L into K chunks, a first kernel runs every chunk but the last from a
//     zero state and records its end state hloc_c and sum of delta; a carry
//     kernel composes the affine maps h -> P_c h + hloc_c with
//     P_c = exp(A * sum(delta over chunk c)) in chunk order, one (b, d, n)
//     per thread; the main kernel then runs every chunk from its true
//     entering state.  The first kernel
//     needs no readout, so it carries g = A*h instead of h:
//     g = fma(a, g, fma(a, B*x, -B*x)), one multiply per element fewer, and
//     converts back (h = g/A) once at the end of the chunk.
//   * A == 0 (which the ZOH formula reaches only as a limit) switches the
//     affected wave to a form with that limit, Bbar = delta * B.
//   * Variants (template bit V): A given per channel (one exp2 per step and
//     lane instead of one per state) and the Euler rule Bbar = delta * B.
//   * With the fused prologue the loader computes x = act(conv1d(x_raw) + b)
//     and delta = softplus(delta_raw + bias) on the way into LDS.

#include <type_traits>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {
namespace {

constexpr int kChunkAlign = 16;  // chunks start on a multiple of this many steps
constexpr int kT = 8;            // steps per staged tile
constexpr int kXS = kT + 4;      // floats per channel row of staged x / delta:
                                 // 16-byte aligned rows, conflict-free 16-byte reads
constexpr int kTileBC = kT * kDState;        // B (or C) values per tile
static_assert(kTileBC % kWave == 0, "B/C tile must split evenly over a wave");
// Register budgets: the main pass keeps 5 waves per SIMD resident (the plan
// puts 5 blocks of 4 waves on every CU), the carry pass 4.
constexpr int kMainWavesPerSimd = 5;
constexpr int kCarryWavesPerSimd = 4;
// the fused prologue's loader registers do not fit in 5 waves' budget
constexpr int kFusedWavesPerSimd = 4;

// ZOH coefficients of one (step, state): h' = a*h + b with a = Abar and
// b = Bbar*x.  With q = B*x/A, Bbar*x = (Abar - 1)*q = fma(Abar, q, -q).
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

// Variants of the per-element formula (bits of the template parameter V):
//  kScalarA -- A holds one value per channel, shared by its 16 states
//              (A[d] instead of A[d, n]): one exp2 per (t, d) instead of 16;
//  kEuler   -- Euler-like input term Bbar = delta*B instead of the ZOH
//              (exp(delta*A) - 1)/A * B (paperlens tutorial, selection-section
//              pseudo-code); Abar = exp(delta*A) either way.
constexpr int kScalarA = 1;
constexpr int kEuler = 2;

// Per-lane constants: A*log2(e) and 1/A for this wave's states.
template <int NPL, int V = 0>
__device__ __forceinline__ bool load_A(const float* __restrict__ A, int d, int n0,
                                       float (&A2)[NPL], float (&iA)[NPL]) {
  bool zero = false;
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const float av = (V & kScalarA) ? A[d] : A[(size_t)d * kDState + n0 + k];
    A2[k] = av * kLog2e;
    iA[k] = 1.0f / av;
    zero |= (av == 0.0f);
  }
  return zero;
}

// Coefficients of one (step, state) for any variant (unpipelined form).
template <int V, bool ZERO_A>
__device__ __forceinline__ void step_coef(float ds, float xs, float Bn, float A2, float iA,
                                          float& a, float& b) {
  if constexpr ((V & kEuler) != 0) {
    a = fast_exp2(ds * A2);
    b = ds * xs * Bn;
  } else {
    zoh_coef<ZERO_A>(ds, Bn * xs, A2, iA, a, b);
  }
}

// Rows [t_begin, t_end) of one batch row of an [b, L, dim] tensor as a buffer.
template <typename IO>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const IO* p, int b, int64_t seqlen,
                                                            int dim, int64_t t_begin,
                                                            int64_t t_end) {
  const size_t first = ((size_t)b * seqlen + t_begin) * dim;
  return make_rsrc(p + first, (uint32_t)((size_t)(t_end - t_begin) * dim * sizeof(IO)));
}

// Raw (undecoded) I/O element as loaded: bf16 bits in the low half, or fp32 bits.
template <typename IO> struct Raw;
template <> struct Raw<float> {
  __device__ __forceinline__ static uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t v,
                                                  uint32_t s) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, v, s, 0);
  }
  __device__ __forceinline__ static float f(uint32_t v) { return __builtin_bit_cast(float, v); }
  // Write as fp32 into an LDS slot.
  __device__ __forceinline__ static void put(float* slot, uint32_t v) {
    *slot = __builtin_bit_cast(float, v);
  }
};
template <> struct Raw<bf16> {
  __device__ __forceinline__ static uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t v,
                                                  uint32_t s) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, v, s, 0);
  }
  __device__ __forceinline__ static float f(uint32_t v) { return bf16_bits_to_f32(v); }
  // The bf16 bits become the upper half of the fp32 slot; its lower half is
  // zero (cleared at kernel start, never written), so the slot holds the
  // exact fp32 value.
  __device__ __forceinline__ static void put(float* slot, uint32_t v) {
    reinterpret_cast<uint16_t*>(slot)[1] = (uint16_t)v;
  }
};

// Stores of y: one value, or two values rounded together (bf16: one
// v_cvt_pk_bf16_f32, then the two halves to their rows).
template <typename IO> struct Out;
template <> struct Out<float> {
  __device__ __forceinline__ static void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
  }
  __device__ __forceinline__ static void store2(float v0, float v1, __amdgpu_buffer_rsrc_t r,
                                                uint32_t voff, uint32_t s0, uint32_t s1) {
    store(v0, r, voff, s0);
    store(v1, r, voff, s1);
  }
};
template <> struct Out<bf16> {
  __device__ __forceinline__ static uint32_t pack(float v0, float v1) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const v2bf p = __builtin_convertvector((v2f){v0, v1}, v2bf);
    return __builtin_bit_cast(uint32_t, p);
  }
  __device__ __forceinline__ static void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pack(v, v), r, voff, soff, 0);
  }
  __device__ __forceinline__ static void store2(float v0, float v1, __amdgpu_buffer_rsrc_t r,
                                                uint32_t voff, uint32_t s0, uint32_t s1) {
    const uint32_t p = pack(v0, v1);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)p, r, voff, s0, 0);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(p >> 16), r, voff, s1, 0);
  }
};

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time loop).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Keeps the computation of v at this point of the program: an empty asm
// statement that takes v in a VGPR and may change it.  Code motion before
// instruction scheduling would otherwise sink the exp2s and input terms of
// the next step down to their uses, or hoist every LDS read of a tile to its
// top, and either way the live ranges (and VGPR count) grow.
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

// NPL consecutive floats of a wave-uniform LDS address (broadcast read).
template <int NPL>
__device__ __forceinline__ void read_n(const float* p, float (&v)[NPL]) {
  if constexpr (NPL % 4 == 0) {
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q) {
      const float4 w = reinterpret_cast<const float4*>(p)[q];
      v[4 * q] = w.x;
      v[4 * q + 1] = w.y;
      v[4 * q + 2] = w.z;
      v[4 * q + 3] = w.w;
    }
  } else if constexpr (NPL == 2) {
    const float2 w = reinterpret_cast<const float2*>(p)[0];
    v[0] = w.x;
    v[1] = w.y;
  } else {
    v[0] = p[0];
  }
}

// kT floats of one staged row (16-byte aligned) into registers.
__device__ __forceinline__ void read_row(const float* p, float (&v)[kT]) {
#pragma unroll
  for (int q = 0; q < kT / 4; ++q) {
    const float4 w = reinterpret_cast<const float4*>(p)[q];
    v[4 * q] = w.x;
    v[4 * q + 1] = w.y;
    v[4 * q + 2] = w.z;
    v[4 * q + 3] = w.w;
  }
}

// Entries [h0, h0 + kT/2) of one staged row into the same entries of v.
__device__ __forceinline__ void read_half(const float* p, float (&v)[kT], int h0) {
#pragma unroll
  for (int q = h0 / 4; q < (h0 + kT / 2) / 4; ++q) {
    const float4 w = reinterpret_cast<const float4*>(p)[q];
    v[4 * q] = w.x;
    v[4 * q + 1] = w.y;
    v[4 * q + 2] = w.z;
    v[4 * q + 3] = w.w;
  }
}

struct Chunk {
  int lane, g, b, c, d;
  bool active;
  int64_t t_begin, t_end;
};

// Coordinates of this thread's block: chunk c of batch row b, the 64
// channels of group blockIdx.x.
__device__ __forceinline__ Chunk chunk_coords(int dim, int64_t seqlen, int64_t chunk_len, int c,
                                              int b) {
  Chunk k;
  k.lane = threadIdx.x % kWave;
  k.g = wave_id();
  k.b = b;
  k.c = c;
  const int draw = blockIdx.x * kWave + k.lane;
  k.active = draw < dim;
  k.d = k.active ? draw : dim - 1;
  k.t_begin = (int64_t)k.c * chunk_len;
  k.t_end = min(seqlen, k.t_begin + chunk_len);
  return k;
}

// Rows of one chunk of a [b, L, 16] tensor (B or C) as a buffer.
template <typename IO>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bc_rsrc(const IO* p, const Chunk& k,
                                                          int64_t seqlen) {
  const size_t first = ((size_t)k.b * seqlen + k.t_begin) * kDState;
  return make_rsrc(p + first, (uint32_t)((size_t)(k.t_end - k.t_begin) * kDState * sizeof(IO)));
}

// ---------------------------------------------------------------------------
// Staging of input tiles through LDS.
// ---------------------------------------------------------------------------

// One pipeline stage: x and delta as [channel][kXS] rows, B and C as
// [step][state].  WITH_C: the main pass also stages C.
template <bool WITH_C>
struct Stage {
  float x[kWave * kXS];
  float d[kWave * kXS];
  float b[kTileBC];
  float c[WITH_C ? kTileBC : 4];
};

// The fetch of one tile is shared evenly by the G waves of the block.  The
// tile has 2*kT rows of 64 channels (x at steps 0..kT-1, then delta) and
// NBC*kTileBC values of B (and C, when staged); wave g fetches rows
// r = g + G*j and the 64-value pieces u = g + G*j of the B/C values.
template <int G, int NBC>
struct Share {
  static constexpr int kRows = 2 * kT / G;                     // rows per wave
  static constexpr int kPieces = NBC * kTileBC / kWave;        // 64-value pieces per tile
  static constexpr int kBC = (kPieces + G - 1) / G;            // pieces per wave (at most)
  static_assert(2 * kT % G == 0, "rows must split evenly over the waves");
};

template <int G, int NBC>
struct TileRaw {
  uint32_t row[Share<G, NBC>::kRows];
  uint32_t bc[Share<G, NBC>::kBC];
};

// Per-lane constants of the prologue (fused scan only).
struct LanePrologue {
  float w[4];  // taps for steps t-3 .. t (zero-padded when d_conv < 4)
  float cb, db;
  bool silu;
};

__device__ __forceinline__ LanePrologue lane_prologue(const Prologue& pro, int d) {
  LanePrologue lp;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int u = k - (4 - pro.d_conv);  // user tap index
    lp.w[k] = u >= 0 ? pro.conv_w[(size_t)d * pro.d_conv + u] : 0.0f;
  }
  lp.cb = pro.conv_b ? pro.conv_b[d] : 0.0f;
  lp.db = pro.delta_bias ? pro.delta_bias[d] : 0.0f;
  lp.silu = pro.conv_silu != 0;
  return lp;
}

// x = act(conv_b + sum_k w_k x_raw[t - 3 + k]) for the 4 steps xs = x_raw[t-3 .. t].
__device__ __forceinline__ float prologue_conv(const LanePrologue& lp, const float (&xs)[4]) {
  float acc = lp.cb;
#pragma unroll
  for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(lp.w[k], xs[k], acc);
  return lp.silu ? silu(acc) : acc;
}

// softplus(v) = log(1 + exp(v)) in fp32.  log1p(e) with e = exp(v) uses the
// series e - e^2/2 + e^3/3 - e^4/4 + e^5/5 when e < 2^-7 (truncation below
// 2^-29 relative) and log(1 + e) through the hardware log2 otherwise; above
// v = 20 the result is v to fp32 precision.
__device__ __forceinline__ float softplus_f32(float v) {
  const float e = fast_exp2(v * kLog2e);
  float r;
  if (e < 0.0078125f) {
    r = e * __builtin_fmaf(e, __builtin_fmaf(e, __builtin_fmaf(e, __builtin_fmaf(e, 0.2f, -0.25f),
                                                               0.33333334f), -0.5f), 1.0f);
  } else {
    r = __builtin_amdgcn_logf(1.0f + e) * 0.6931471805599453f;
  }
  return v > 20.0f ? v : r;
}

template <typename IO, int G, bool WITH_C>
struct Loader {
  static constexpr int NBC = WITH_C ? 2 : 1;
  using S = Share<G, NBC>;
  using RawTile = TileRaw<G, NBC>;
  __amdgpu_buffer_rsrc_t rx, rd, rb, rc;
  uint32_t voff_row, row_bytes;
  int g;

  __device__ __forceinline__ void init(const IO* x, const IO* delta, const IO* B, const IO* C,
                                       int64_t seqlen, int dim, const Chunk& k,
                                       const LanePrologue&) {
    rx = rows_rsrc(x, k.b, seqlen, dim, k.t_begin, k.t_end);
    rd = rows_rsrc(delta, k.b, seqlen, dim, k.t_begin, k.t_end);
    rb = bc_rsrc(B, k, seqlen);
    rc = bc_rsrc(C, k, seqlen);
    voff_row = (uint32_t)k.d * sizeof(IO);
    row_bytes = (uint32_t)dim * sizeof(IO);
    g = k.g;
  }

  // Global loads of this wave's share of the tile starting at step s0.
  __device__ __forceinline__ void issue(TileRaw<G, NBC>& r, int s0, int lane) const {
#pragma unroll
    for (int j = 0; j < S::kRows; ++j) {
      const int row = g + G * j;  // < 2*kT
      const bool is_d = row >= kT;
      const int s = is_d ? row - kT : row;
      r.row[j] = Raw<IO>::load(is_d ? rd : rx, voff_row, (uint32_t)(s0 + s) * row_bytes);
    }
#pragma unroll
    for (int j = 0; j < S::kBC; ++j) {
      const int piece = min(g + G * j, S::kPieces - 1);  // duplicates are not stored
      const bool is_c = piece * kWave >= kTileBC;
      const int v = piece * kWave - (is_c ? kTileBC : 0) + lane;
      r.bc[j] = Raw<IO>::load(is_c ? rc : rb, (uint32_t)(v * sizeof(IO)),
                              (uint32_t)s0 * kDState * sizeof(IO));
    }
  }

  // Write this wave's share of a tile fetched by issue() into an LDS stage.
  __device__ __forceinline__ void put(const TileRaw<G, NBC>& r, Stage<WITH_C>& st,
                                      int lane) const {
#pragma unroll
    for (int j = 0; j < S::kRows; ++j) {
      const int row = g + G * j;
      const bool is_d = row >= kT;
      const int s = is_d ? row - kT : row;
      Raw<IO>::put((is_d ? st.d : st.x) + lane * kXS + s, r.row[j]);
    }
#pragma unroll
    for (int j = 0; j < S::kBC; ++j) {
      const int piece = g + G * j;
      if (piece < S::kPieces) {
        const bool is_c = piece * kWave >= kTileBC;
        const int v = piece * kWave - (is_c ? kTileBC : 0) + lane;
        Raw<IO>::put((is_c ? st.c : st.b) + v, r.bc[j]);
      }
    }
  }

  // x and delta of one step (ragged end of a chunk), straight from memory.
  __device__ __forceinline__ void step(int s, float& xs, float& ds) const {
    const uint32_t so = (uint32_t)s * row_bytes;
    xs = buf<IO>::load(rx, voff_row, so);
    ds = buf<IO>::load(rd, voff_row, so);
  }
};

// Loader of the fused scan: the tile's x and delta are computed from x_raw
// and delta_raw on the way into LDS.  Wave g produces the kT/G consecutive
// steps [g*kT/G, (g+1)*kT/G) of the tile for its 64 channels: it fetches
// those steps of delta_raw and of x_raw with the 3 steps before them (the
// convolution's reach; zeros before the start of the sequence), applies the
// causal convolution, its bias and optional SiLU, and softplus(delta_raw +
// bias).  B and C pieces are shared out as in Loader.
template <int G, int NBC>
struct FusedRaw {
  static constexpr int kSteps = kT / G;
  uint32_t xr[kSteps + 3];
  uint32_t dr[kSteps];
  uint32_t bc[Share<G, NBC>::kBC];
};

template <typename IO, int G, bool WITH_C>
struct FusedLoader {
  static constexpr int NBC = WITH_C ? 2 : 1;
  static constexpr int kSteps = kT / G;
  static_assert(G <= kT, "the fused loader gives every wave at least one step");
  using S = Share<G, NBC>;
  using RawTile = FusedRaw<G, NBC>;
  __amdgpu_buffer_rsrc_t rx, rd, rb, rc;
  uint32_t voff_row, row_bytes;
  int g, xshift;      // xshift: rows of x_raw kept before the chunk start (0..3)
  int64_t t_begin;
  LanePrologue lp;

  __device__ __forceinline__ void init(const IO* x_raw, const IO* delta_raw, const IO* B,
                                       const IO* C, int64_t seqlen, int dim, const Chunk& k,
                                       const LanePrologue& lpin) {
    const int64_t xb = k.t_begin >= 3 ? k.t_begin - 3 : 0;
    xshift = (int)(k.t_begin - xb);
    rx = rows_rsrc(x_raw, k.b, seqlen, dim, xb, k.t_end);
    rd = rows_rsrc(delta_raw, k.b, seqlen, dim, k.t_begin, k.t_end);
    rb = bc_rsrc(B, k, seqlen);
    rc = bc_rsrc(C, k, seqlen);
    voff_row = (uint32_t)k.d * sizeof(IO);
    row_bytes = (uint32_t)dim * sizeof(IO);
    g = k.g;
    t_begin = k.t_begin;
    lp = lpin;
  }

  // x_raw at step `rel` of the chunk (rel >= -3); zero before the sequence.
  __device__ __forceinline__ uint32_t load_x(int rel) const {
    const bool ok = t_begin + rel >= 0;
    return Raw<IO>::load(rx, ok ? voff_row : 0x80000000u,
                         ok ? (uint32_t)(rel + xshift) * row_bytes : 0u);
  }

  __device__ __forceinline__ float conv(const float (&xs)[4]) const { return prologue_conv(lp, xs); }

  __device__ __forceinline__ void issue(RawTile& r, int s0, int lane) const {
    const int t0 = s0 + g * kSteps;
#pragma unroll
    for (int j = 0; j < kSteps + 3; ++j) r.xr[j] = load_x(t0 - 3 + j);
#pragma unroll
    for (int j = 0; j < kSteps; ++j)
      r.dr[j] = Raw<IO>::load(rd, voff_row, (uint32_t)(t0 + j) * row_bytes);
#pragma unroll
    for (int j = 0; j < S::kBC; ++j) {
      const int piece = min(g + G * j, S::kPieces - 1);
      const bool is_c = piece * kWave >= kTileBC;
      const int v = piece * kWave - (is_c ? kTileBC : 0) + lane;
      r.bc[j] = Raw<IO>::load(is_c ? rc : rb, (uint32_t)(v * sizeof(IO)),
                              (uint32_t)s0 * kDState * sizeof(IO));
    }
  }

  __device__ __forceinline__ void put(const RawTile& r, Stage<WITH_C>& st, int lane) const {
    float* xrow = st.x + lane * kXS + g * kSteps;
    float* drow = st.d + lane * kXS + g * kSteps;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const float xs[4] = {Raw<IO>::f(r.xr[j]), Raw<IO>::f(r.xr[j + 1]), Raw<IO>::f(r.xr[j + 2]),
                           Raw<IO>::f(r.xr[j + 3])};
      xrow[j] = conv(xs);
      drow[j] = softplus_f32(Raw<IO>::f(r.dr[j]) + lp.db);
    }
#pragma unroll
    for (int j = 0; j < S::kBC; ++j) {
      const int piece = g + G * j;
      if (piece < S::kPieces) {
        const bool is_c = piece * kWave >= kTileBC;
        const int v = piece * kWave - (is_c ? kTileBC : 0) + lane;
        Raw<IO>::put((is_c ? st.c : st.b) + v, r.bc[j]);
      }
    }
  }

  // x and delta of one step (ragged end of a chunk), computed from memory.
  __device__ __forceinline__ void step(int s, float& xs, float& ds) const {
    float w4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w4[k] = Raw<IO>::f(load_x(s - 3 + k));
    xs = conv(w4);
    ds = softplus_f32(Raw<IO>::f(Raw<IO>::load(rd, voff_row, (uint32_t)s * row_bytes)) + lp.db);
  }
};

// Clear both stages (bf16 inputs rely on zero lower halves of the slots).
template <typename IO, bool WITH_C>
__device__ __forceinline__ void clear_stages(Stage<WITH_C>* st, int nthreads) {
  if constexpr (std::is_same<IO, bf16>::value) {
    static_assert(sizeof(Stage<WITH_C>) % sizeof(float4) == 0, "stage size");
    float4* p = reinterpret_cast<float4*>(st);
    constexpr int n = (int)(2 * sizeof(Stage<WITH_C>) / sizeof(float4));
    for (int i = threadIdx.x; i < n; i += nthreads) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ---------------------------------------------------------------------------
// Main scan: one chunk of 64 channels x all 16 states per block.
// ---------------------------------------------------------------------------
template <int G>
struct MainSmem {
  Stage<true> st[2];
  float part[2][kT * G * kWave];  // [buffer][step][wave][lane]
};

template <typename IO, int G, bool HAS_Z, bool ZERO_A, bool FUSED, int V>
__device__ __forceinline__ void scan_chunk(const IO* __restrict__ x, const IO* __restrict__ delta,
                                           const IO* __restrict__ B, const IO* __restrict__ C,
                                           const IO* __restrict__ z, IO* __restrict__ y,
                                           float Dd, int64_t seqlen, int dim, const Chunk& k,
                                           MainSmem<G>& sm, const float (&A2)[kDState / G],
                                           const float (&iA)[kDState / G],
                                           float (&h)[kDState / G], const LanePrologue& lp) {
  constexpr int NPL = kDState / G;
  constexpr int ZT = (kT + G - 1) / G;        // steps of a tile this wave finishes (at most)
  const int lane = k.lane, g = k.g, n0 = g * NPL;
  const __amdgpu_buffer_rsrc_t rz = rows_rsrc(HAS_Z ? z : x, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t ry = rows_rsrc(y, k.b, seqlen, dim, k.t_begin, k.t_end);
  const uint32_t voff = (uint32_t)k.d * sizeof(IO);
  // lanes past the last channel store out of the buffer's range (dropped)
  const uint32_t voff_y = k.active ? voff : 0x80000000u;
  const uint32_t row_bytes = (uint32_t)dim * sizeof(IO);
  const int nsteps = (int)(k.t_end - k.t_begin);
  const int nfull = nsteps / kT;

  using LD = std::conditional_t<FUSED, FusedLoader<IO, G, true>, Loader<IO, G, true>>;
  using Raw2 = typename LD::RawTile;
  LD ld;
  ld.init(x, delta, B, C, seqlen, dim, k, lp);

  // z of the steps this wave finishes in tile `tidx` (clamped past the end)
  auto issue_z = [&](uint32_t (&zr)[ZT], int tidx) {
    if constexpr (HAS_Z) {
      const int s0 = min(tidx, nfull - 1) * kT;
#pragma unroll
      for (int j = 0; j < ZT; ++j)
        zr[j] = Raw<IO>::load(rz, voff, (uint32_t)min(s0 + g + j * G, nsteps - 1) * row_bytes);
    }
  };

  int pb = 0;
  // One tile: compute from stage `cur`, write the next tile's data into the
  // other stage, barrier, then finish this wave's steps of the tile.
  auto tile = [&](int tidx, int cur, Raw2& rissue, const Raw2& rput,
                  const uint32_t (&zuse)[ZT], uint32_t (&znext)[ZT]) {
    const int s0 = tidx * kT;
    ld.issue(rissue, min(tidx + 2, nfull - 1) * kT, lane);
    issue_z(znext, tidx + 1);
    const Stage<true>& st = sm.st[cur];
    // x and delta of the tile, read in two halves (the second half once the
    // first is no longer needed) to keep the register count down
    float xv[kT], dv[kT], xe[ZT];
    read_half(st.x + lane * kXS, xv, 0);
    read_half(st.d + lane * kXS, dv, 0);
#pragma unroll
    for (int j = 0; j < ZT; ++j) xe[j] = st.x[lane * kXS + min(g + j * G, kT - 1)];
    float* pw = sm.part[pb] + g * kWave + lane;  // + s * G * kWave for step s

    // B and C of step s are read from LDS two steps before their use; the
    // exp2s and input terms are formed one step before (all exp2s of a step
    // first, so their latency overlaps the input terms).
    float bq[2][NPL], cq[2][NPL];
    auto fetch = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      read_n<NPL>(st.b + s * kDState + n0, bq[s & 1]);
      read_n<NPL>(st.c + s * kDState + n0, cq[s & 1]);
    };
    float ca[2][NPL], cb[2][NPL], cc[2][NPL];
    auto coefs = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr ((V & kScalarA) != 0) {
        // one exp2 and one input term per step, shared by the wave's states
        float a = fast_exp2(dv[s] * A2[0]);
        float c;  // Bbar*x / B
        if constexpr ((V & kEuler) != 0) {
          c = dv[s] * xv[s];
        } else if constexpr (!ZERO_A) {
          const float q = xv[s] * iA[0];
          c = __builtin_fmaf(a, q, -q);
        } else {
          c = (__builtin_isinf(iA[0]) ? dv[s] : (a - 1.0f) * iA[0]) * xv[s];
        }
        pin(a);
#pragma unroll
        for (int n = 0; n < NPL; ++n) {
          ca[s & 1][n] = a;
          cb[s & 1][n] = c * bq[s & 1][n];
          pin(cb[s & 1][n]);
          cc[s & 1][n] = cq[s & 1][n];
        }
      } else {
#pragma unroll
        for (int n = 0; n < NPL; ++n) {
          ca[s & 1][n] = fast_exp2(dv[s] * A2[n]);
          pin(ca[s & 1][n]);
        }
        const float dx = dv[s] * xv[s];  // Euler: Bbar*x = (delta*x) * B
#pragma unroll
        for (int n = 0; n < NPL; ++n) {
          const float bx = bq[s & 1][n] * xv[s];
          const float a = ca[s & 1][n];
          if constexpr ((V & kEuler) != 0) {
            cb[s & 1][n] = dx * bq[s & 1][n];
          } else if constexpr (!ZERO_A) {
            const float q = bx * iA[n];
            cb[s & 1][n] = __builtin_fmaf(a, q, -q);
          } else {
            cb[s & 1][n] = (__builtin_isinf(iA[n]) ? dv[s] : (a - 1.0f) * iA[n]) * bx;
          }
          pin(cb[s & 1][n]);
          cc[s & 1][n] = cq[s & 1][n];
        }
      }
    };
    fetch(std::integral_constant<int, 0>{});
    fetch(std::integral_constant<int, 1>{});
    coefs(std::integral_constant<int, 0>{});
    static_for<kT>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s + 1 < kT) coefs(std::integral_constant<int, s + 1>{});
      if constexpr (s + 2 == kT / 2) {
        read_half(st.x + lane * kXS, xv, kT / 2);
        read_half(st.d + lane * kXS, dv, kT / 2);
      }
      if constexpr (s + 2 < kT) fetch(std::integral_constant<int, s + 2>{});
      h[0] = __builtin_fmaf(ca[s & 1][0], h[0], cb[s & 1][0]);
      float acc = cc[s & 1][0] * h[0];
#pragma unroll
      for (int n = 1; n < NPL; ++n) {
        h[n] = __builtin_fmaf(ca[s & 1][n], h[n], cb[s & 1][n]);
        acc = __builtin_fmaf(cc[s & 1][n], h[n], acc);
      }
      pin(acc);
      pw[s * G * kWave] = acc;
    });
    ld.put(rput, sm.st[cur ^ 1], lane);
    __syncthreads();
    // epilogue: sum of the G partials, skip term, gate, store
    const float* pr = sm.part[pb] + lane;
    float ps[ZT][G];
#pragma unroll
    for (int j = 0; j < ZT; ++j) {
      const int s = min(g + j * G, kT - 1);
#pragma unroll
      for (int w = 0; w < G; ++w) ps[j][w] = pr[(s * G + w) * kWave];
    }
    float yv[ZT];
#pragma unroll
    for (int j = 0; j < ZT; ++j) {
      float sum = ps[j][0];
#pragma unroll
      for (int w = 1; w < G; ++w) sum += ps[j][w];
      const float pre = __builtin_fmaf(Dd, xe[j], sum);
      if constexpr (HAS_Z)
        yv[j] = pre * silu(Raw<IO>::f(zuse[j]));
      else
        yv[j] = pre;
    }
    if constexpr (ZT == 2 && kT == 2 * G) {
      Out<IO>::store2(yv[0], yv[1], ry, voff_y, (uint32_t)(s0 + g) * row_bytes,
                      (uint32_t)(s0 + g + G) * row_bytes);
    } else {
#pragma unroll
      for (int j = 0; j < ZT; ++j) {
        const int s = g + j * G;
        if (kT % G != 0 && s >= kT) break;
        Out<IO>::store(yv[j], ry, voff_y, (uint32_t)(s0 + s) * row_bytes);
      }
    }
    pb ^= 1;
  };

  if (nfull > 0) {
    Raw2 ra, rb;
    uint32_t za[ZT], zb[ZT];
    ld.issue(ra, 0, lane);
    ld.issue(rb, min(1, nfull - 1) * kT, lane);
    issue_z(za, 0);
    ld.put(ra, sm.st[0], lane);
    __syncthreads();
    int i = 0;
    for (; i + 2 <= nfull; i += 2) {
      tile(i, 0, ra, rb, za, zb);
      tile(i + 1, 1, rb, ra, zb, za);
    }
    if (i < nfull) tile(i, 0, ra, rb, za, zb);
  }

  // ragged end of the chunk: one step at a time from global memory
  const __amdgpu_buffer_rsrc_t rbb = bc_rsrc(B, k, seqlen);
  const __amdgpu_buffer_rsrc_t rcc = bc_rsrc(C, k, seqlen);
  for (int s0 = nfull * kT; s0 < nsteps; ++s0) {
    const uint32_t so = (uint32_t)s0 * row_bytes;
    float xs, ds;
    ld.step(s0, xs, ds);
    const uint32_t bo = (uint32_t)(s0 * kDState + n0) * sizeof(IO);
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < NPL; ++n) {
      const float Bn = buf<IO>::load(rbb, bo + n * sizeof(IO), 0);
      const float Cn = buf<IO>::load(rcc, bo + n * sizeof(IO), 0);
      float a, b;
      step_coef<V, ZERO_A>(ds, xs, Bn, A2[n], iA[n], a, b);
      h[n] = __builtin_fmaf(a, h[n], b);
      acc = __builtin_fmaf(Cn, h[n], acc);
    }
    float* pbuf = sm.part[pb];
    pbuf[g * kWave + lane] = acc;
    __syncthreads();
    if (g == 0) {
      float sum = pbuf[lane];
#pragma unroll
      for (int w = 1; w < G; ++w) sum += pbuf[w * kWave + lane];
      const float pre = __builtin_fmaf(Dd, xs, sum);
      const float yv = HAS_Z ? pre * silu(buf<IO>::load(rz, voff, so)) : pre;
      Out<IO>::store(yv, ry, voff_y, so);
    }
    pb ^= 1;
  }
}

// Main pass of one block: its 64 channels over chunk k from the state
// `hinit` (nullable = zero state; [.., 16] rows of the block's channels),
// writing y and, when `hout` is given, the state at the end of the chunk.
template <typename IO, int G, bool HAS_Z, bool FUSED, int V>
__device__ __forceinline__ void main_block(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, const IO* __restrict__ C, const float* __restrict__ Dskip,
    const IO* __restrict__ z, IO* __restrict__ y, const float* hinit, float* hout,
    int64_t seqlen, int dim, const Chunk& k, MainSmem<G>& sm, const Prologue& pro) {
  constexpr int NPL = kDState / G;
  const int n0 = k.g * NPL;
  clear_stages<IO, true>(sm.st, kWave * G);

  float A2[NPL], iA[NPL], h[NPL];
  const bool zero = load_A<NPL, V>(A, k.d, n0, A2, iA);
#pragma unroll
  for (int j = 0; j < NPL; ++j) h[j] = hinit ? hinit[j] : 0.0f;
  const float Dd = Dskip ? Dskip[k.d] : 0.0f;
  LanePrologue lp{};
  if constexpr (FUSED) lp = lane_prologue(pro, k.d);
  __syncthreads();  // stages cleared

  if (__builtin_amdgcn_ballot_w64(zero) != 0)
    scan_chunk<IO, G, HAS_Z, true, FUSED, V>(x, delta, B, C, z, y, Dd, seqlen, dim, k, sm, A2,
                                             iA, h, lp);
  else
    scan_chunk<IO, G, HAS_Z, false, FUSED, V>(x, delta, B, C, z, y, Dd, seqlen, dim, k, sm, A2,
                                              iA, h, lp);

  if (hout && k.active) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) hout[j] = h[j];
  }
}

// ---------------------------------------------------------------------------
// Main pass, wave-independent form (4 waves per group, A per (channel,
// state); ZOH or Euler rule; with or without the fused prologue).  Wave w of
// the block owns the 16 channels d0 + 16w .. d0 + 16w + 15 with all 16
// states: lane l holds channel c = l % 16 of the wave and the states
// 4r .. 4r + 3 of its row r = l / 16 (rows of 16 lanes).  Each wave stages
// its own tiles of x, delta, B and C through its own LDS region (x and delta
// as [channel][step], B and C as [step][state]; the row's 16 lanes read the
// same B/C values), so no barrier couples the block's waves.  Readout: per
// step every lane forms its 4-state partial; after four steps the partials
// of the four rows are transposed through the wave's own LDS area and
// summed, (rows 0 + 1) + (rows 2 + 3), which leaves in row r the total of
// the group's step r.  Row r then finishes that step (skip term, gate,
// store): each lane stores two steps of a tile.
// ---------------------------------------------------------------------------
constexpr int kWCh = kWave / 4;  // channels per wave

struct WStage {
  float x[kWCh * kXS];
  float d[kWCh * kXS];
  float b[kTileBC];
  float c[kTileBC];
};
constexpr int kTrRow = 20;  // floats per channel of the readout transpose (16-byte rows)
struct alignas(16) WSmem {
  WStage st[4][2];             // [wave][stage]
  float tr[4][kWCh * kTrRow];  // [wave] readout transpose
};

// Lane coordinates of the wave-independent form.
struct WLane {
  int c, r;     // channel of the wave (0..15), row (0..3)
  int d;        // channel index (clamped to dim - 1 past the end)
  bool active;  // d < dim
};

__device__ __forceinline__ WLane wlane(int dim) {
  WLane w;
  const int lane = threadIdx.x % kWave;
  w.c = lane % kWCh;
  w.r = lane / kWCh;
  const int draw = blockIdx.x * kWave + wave_id() * kWCh + w.c;
  w.active = draw < dim;
  w.d = w.active ? draw : dim - 1;
  return w;
}

// Sum over the four rows, transposed: p[s] is this lane's partial of step s;
// returns in row r the total of step r over the rows of this lane's column,
// as (rows 0 + 1) + (rows 2 + 3).  Through the wave's own LDS area: lane
// (c, r) writes its partial of step s to tw[c][4s + r], then reads the four
// rows' partials of step r, tw[c][4r .. 4r + 3].  The wave's LDS accesses
// execute in program order, and these writes and reads are float accesses
// of the same array, so the compiler keeps their order too.
__device__ __forceinline__ float rows_transpose_sum(float* tw, const WLane& w, float p0,
                                                    float p1, float p2, float p3) {
  float* wp = tw + w.c * kTrRow + w.r;
  wp[0] = p0;
  wp[4] = p1;
  wp[8] = p2;
  wp[12] = p3;
  const float* rp = tw + w.c * kTrRow + 4 * w.r;
  return (rp[0] + rp[1]) + (rp[2] + rp[3]);
}

// Raw values of one tile fetched by a lane: x and delta at steps r and r + 4
// of its channel; B and C as two consecutive tile values each (bf16: one
// 32-bit load; fp32: two loads).
template <typename IO> struct WRaw {
  static constexpr int kBC = sizeof(IO) == 2 ? 1 : 2;
  uint32_t x[2], d[2];
  uint32_t b[kBC], c[kBC];
};

template <typename IO, bool WITH_C = true>
struct WLoader {
  using RawTile = WRaw<IO>;
  __amdgpu_buffer_rsrc_t rx, rd, rb, rc;
  uint32_t voff, voff_c, row_bytes;  // voff: row r and channel d; voff_c: channel d (bytes)

  __device__ __forceinline__ void init(const IO* x, const IO* delta, const IO* B, const IO* C,
                                       int64_t seqlen, int dim, const Chunk& k, const WLane& w,
                                       const LanePrologue&) {
    rx = rows_rsrc(x, k.b, seqlen, dim, k.t_begin, k.t_end);
    rd = rows_rsrc(delta, k.b, seqlen, dim, k.t_begin, k.t_end);
    rb = bc_rsrc(B, k, seqlen);
    rc = bc_rsrc(C, k, seqlen);
    row_bytes = (uint32_t)dim * sizeof(IO);
    voff_c = (uint32_t)w.d * sizeof(IO);
    voff = (uint32_t)w.r * row_bytes + voff_c;
  }

  // x and delta of step s (uniform), straight from memory.
  __device__ __forceinline__ void step(int s, float& xs, float& ds) const {
    const uint32_t so = (uint32_t)s * row_bytes;
    xs = buf<IO>::load(rx, voff_c, so);
    ds = buf<IO>::load(rd, voff_c, so);
  }

  // x of step g0 + r (this lane's row), straight from memory.
  __device__ __forceinline__ float x_row(int g0) const {
    return buf<IO>::load(rx, voff, (uint32_t)g0 * row_bytes);
  }

  // Loads of the (full) tile starting at step s0 of the chunk.
  __device__ __forceinline__ void issue(WRaw<IO>& t, int s0, int lane) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t so = (uint32_t)(s0 + 4 * j) * row_bytes;
      t.x[j] = Raw<IO>::load(rx, voff, so);
      t.d[j] = Raw<IO>::load(rd, voff, so);
    }
    const uint32_t bo = (uint32_t)s0 * kDState * sizeof(IO);
    if constexpr (sizeof(IO) == 2) {
      t.b[0] = __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)lane * 4u, bo, 0);
      if constexpr (WITH_C)
        t.c[0] = __builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)lane * 4u, bo, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        t.b[e] = __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)(2 * lane + e) * 4u, bo, 0);
        if constexpr (WITH_C)
          t.c[e] = __builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)(2 * lane + e) * 4u, bo, 0);
      }
    }
  }

  // Write a fetched tile into the wave's LDS stage.  The wave's LDS accesses
  // execute in program order; the empty asm statements with a memory clobber
  // keep the compiler from moving the stage's reads across these writes
  // (with no barrier between them, type-based alias analysis would let it
  // reorder the 16-byte reads and the 4- or 2-byte writes).
  __device__ __forceinline__ void put(const WRaw<IO>& t, WStage& st, const WLane& w,
                                      int lane) const {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      Raw<IO>::put(st.x + w.c * kXS + 4 * j + w.r, t.x[j]);
      Raw<IO>::put(st.d + w.c * kXS + 4 * j + w.r, t.d[j]);
    }
    if constexpr (sizeof(IO) == 2) {
      Raw<IO>::put(st.b + 2 * lane, t.b[0] & 0xffffu);
      Raw<IO>::put(st.b + 2 * lane + 1, t.b[0] >> 16);
      if constexpr (WITH_C) {
        Raw<IO>::put(st.c + 2 * lane, t.c[0] & 0xffffu);
        Raw<IO>::put(st.c + 2 * lane + 1, t.c[0] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        Raw<IO>::put(st.b + 2 * lane + e, t.b[e]);
        if constexpr (WITH_C) Raw<IO>::put(st.c + 2 * lane + e, t.c[e]);
      }
    }
    asm volatile("" ::: "memory");
  }
};

// Loader of the fused scan in the wave-independent form: lane (c, r) produces
// x = act(conv1d(x_raw) + b) and delta = softplus(delta_raw + bias) of the
// two consecutive steps 2r and 2r + 1 of each tile for its channel, from
// x_raw of steps 2r - 3 .. 2r + 1 (zero before the start of the sequence)
// and delta_raw of its two steps; B and C as in WLoader.
template <typename IO> struct WFusedRaw {
  static constexpr int kBC = sizeof(IO) == 2 ? 1 : 2;
  uint32_t xr[5], dr[2];
  uint32_t b[kBC], c[kBC];
};

template <typename IO, bool WITH_C = true>
struct WFusedLoader {
  using RawTile = WFusedRaw<IO>;
  __amdgpu_buffer_rsrc_t rx, rd, rb, rc;
  uint32_t voff, voff_c, row_bytes;
  int xshift, r;     // xshift: rows of x_raw kept before the chunk start (0..3)
  int64_t t_begin;
  LanePrologue lp;

  __device__ __forceinline__ void init(const IO* x_raw, const IO* delta_raw, const IO* B,
                                       const IO* C, int64_t seqlen, int dim, const Chunk& k,
                                       const WLane& w, const LanePrologue& lpin) {
    const int64_t xb = k.t_begin >= 3 ? k.t_begin - 3 : 0;
    xshift = (int)(k.t_begin - xb);
    rx = rows_rsrc(x_raw, k.b, seqlen, dim, xb, k.t_end);
    rd = rows_rsrc(delta_raw, k.b, seqlen, dim, k.t_begin, k.t_end);
    rb = bc_rsrc(B, k, seqlen);
    rc = bc_rsrc(C, k, seqlen);
    row_bytes = (uint32_t)dim * sizeof(IO);
    voff_c = (uint32_t)w.d * sizeof(IO);
    voff = (uint32_t)w.r * row_bytes + voff_c;
    r = w.r;
    t_begin = k.t_begin;
    lp = lpin;
  }

  // x_raw at step `rel` of the chunk (rel >= -3, uniform); zero before the sequence.
  __device__ __forceinline__ uint32_t load_x(int rel) const {
    const bool ok = t_begin + rel >= 0;
    return Raw<IO>::load(rx, ok ? voff_c : 0x80000000u,
                         ok ? (uint32_t)(rel + xshift) * row_bytes : 0u);
  }

  __device__ __forceinline__ void issue(RawTile& t, int s0, int lane) const {
    // rows 2r - 3 .. 2r + 1 of the tile: the row offset is per lane
    const int t0 = s0 + 2 * r;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int rel = t0 - 3 + j;
      const bool ok = t_begin + rel >= 0;
      t.xr[j] = Raw<IO>::load(rx, ok ? voff_c + (uint32_t)(rel + xshift) * row_bytes : 0x80000000u,
                              0u);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      t.dr[j] = Raw<IO>::load(rd, voff_c + (uint32_t)(t0 + j) * row_bytes, 0u);
    const uint32_t bo = (uint32_t)s0 * kDState * sizeof(IO);
    if constexpr (sizeof(IO) == 2) {
      t.b[0] = __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)lane * 4u, bo, 0);
      if constexpr (WITH_C)
        t.c[0] = __builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)lane * 4u, bo, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        t.b[e] = __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)(2 * lane + e) * 4u, bo, 0);
        if constexpr (WITH_C)
          t.c[e] = __builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)(2 * lane + e) * 4u, bo, 0);
      }
    }
  }

  // Compute the tile's x and delta into the wave's LDS stage (memory clobbers
  // as in WLoader::put).
  __device__ __forceinline__ void put(const RawTile& t, WStage& st, const WLane& w,
                                      int lane) const {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float xs[4] = {Raw<IO>::f(t.xr[j]), Raw<IO>::f(t.xr[j + 1]), Raw<IO>::f(t.xr[j + 2]),
                           Raw<IO>::f(t.xr[j + 3])};
      st.x[w.c * kXS + 2 * w.r + j] = prologue_conv(lp, xs);
      st.d[w.c * kXS + 2 * w.r + j] = softplus_f32(Raw<IO>::f(t.dr[j]) + lp.db);
    }
    if constexpr (sizeof(IO) == 2) {
      Raw<IO>::put(st.b + 2 * lane, t.b[0] & 0xffffu);
      Raw<IO>::put(st.b + 2 * lane + 1, t.b[0] >> 16);
      if constexpr (WITH_C) {
        Raw<IO>::put(st.c + 2 * lane, t.c[0] & 0xffffu);
        Raw<IO>::put(st.c + 2 * lane + 1, t.c[0] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        Raw<IO>::put(st.b + 2 * lane + e, t.b[e]);
        if constexpr (WITH_C) Raw<IO>::put(st.c + 2 * lane + e, t.c[e]);
      }
    }
    asm volatile("" ::: "memory");
  }

  // x and delta of step s (uniform), computed from memory.
  __device__ __forceinline__ void step(int s, float& xs, float& ds) const {
    float w4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w4[k] = Raw<IO>::f(load_x(s - 3 + k));
    xs = prologue_conv(lp, w4);
    ds = softplus_f32(Raw<IO>::f(Raw<IO>::load(rd, voff_c, (uint32_t)s * row_bytes)) + lp.db);
  }

  // x of step g0 + r (this lane's row), computed from memory.
  __device__ __forceinline__ float x_row(int g0) const {
    float w4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rel = g0 + r - 3 + k;
      const bool ok = t_begin + rel >= 0;
      w4[k] = Raw<IO>::f(Raw<IO>::load(
          rx, ok ? voff_c + (uint32_t)(rel + xshift) * row_bytes : 0x80000000u, 0u));
    }
    return prologue_conv(lp, w4);
  }
};

template <typename IO, bool HAS_Z, bool ZERO_A, bool FUSED, int V>
__device__ __forceinline__ void scan_chunk_w(const IO* __restrict__ x,
                                             const IO* __restrict__ delta,
                                             const IO* __restrict__ B, const IO* __restrict__ C,
                                             const IO* __restrict__ z, IO* __restrict__ y,
                                             float Dd, int64_t seqlen, int dim, const Chunk& k,
                                             const WLane& w, WStage (&sts)[2], float* tw,
                                             const float (&A2)[4], const float (&iA)[4],
                                             float (&h)[4], const LanePrologue& lp) {
  static_assert((V & kScalarA) == 0, "A per channel uses scan_chunk");
  const int lane = threadIdx.x % kWave;
  const int n0 = 4 * w.r;
  const __amdgpu_buffer_rsrc_t rz = rows_rsrc(HAS_Z ? z : x, k.b, seqlen, dim, k.t_begin, k.t_end);
  const __amdgpu_buffer_rsrc_t ry = rows_rsrc(y, k.b, seqlen, dim, k.t_begin, k.t_end);
  using LD = std::conditional_t<FUSED, WFusedLoader<IO, true>, WLoader<IO, true>>;
  using RawT = typename LD::RawTile;
  LD ld;
  ld.init(x, delta, B, C, seqlen, dim, k, w, lp);
  const uint32_t row_bytes = ld.row_bytes;
  // lanes past the last channel store out of the buffer's range (dropped)
  const uint32_t voff_y = w.active ? ld.voff : 0x80000000u;
  const int nsteps = (int)(k.t_end - k.t_begin);
  const int nfull = nsteps / kT;

  // z of this lane's two steps (r, r + 4) of tile `tidx` (clamped)
  auto issue_z = [&](uint32_t (&zr)[2], int tidx) {
    if constexpr (HAS_Z) {
      const int s0 = min(tidx, nfull - 1) * kT;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        zr[j] = Raw<IO>::load(rz, ld.voff, (uint32_t)(s0 + 4 * j) * row_bytes);
    }
  };

  // Epilogue of step s0 + 4j + r: total S, skip term, gate.
  auto finish = [&](float S, float xe, uint32_t zraw) {
    const float pre = __builtin_fmaf(Dd, xe, S);
    if constexpr (HAS_Z)
      return pre * silu(Raw<IO>::f(zraw));
    else
      return pre;
  };

  auto tile = [&](int tidx, int cur, RawT& rissue, const RawT& rput,
                  const uint32_t (&zuse)[2], uint32_t (&znext)[2]) {
    const int s0 = tidx * kT;
    ld.issue(rissue, min(tidx + 2, nfull - 1) * kT, lane);
    issue_z(znext, tidx + 1);
    const WStage& st = sts[cur];
    float xv[kT], dv[kT];
    read_half(st.x + w.c * kXS, xv, 0);
    read_half(st.d + w.c * kXS, dv, 0);
    float bq[2][4], cq[2][4];
    auto fetch = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      read_n<4>(st.b + s * kDState + n0, bq[s & 1]);
      read_n<4>(st.c + s * kDState + n0, cq[s & 1]);
    };
    float ca[2][4], cb[2][4], cc[2][4];
    auto coefs = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        ca[s & 1][n] = fast_exp2(dv[s] * A2[n]);
        pin(ca[s & 1][n]);
      }
      const float dx = dv[s] * xv[s];  // Euler: Bbar*x = (delta*x) * B
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const float bx = bq[s & 1][n] * xv[s];
        const float a = ca[s & 1][n];
        if constexpr ((V & kEuler) != 0) {
          cb[s & 1][n] = dx * bq[s & 1][n];
        } else if constexpr (!ZERO_A) {
          const float q = bx * iA[n];
          cb[s & 1][n] = __builtin_fmaf(a, q, -q);
        } else {
          cb[s & 1][n] = (__builtin_isinf(iA[n]) ? dv[s] : (a - 1.0f) * iA[n]) * bx;
        }
        pin(cb[s & 1][n]);
        cc[s & 1][n] = cq[s & 1][n];
      }
    };
    float p[4], yv[2];
    fetch(std::integral_constant<int, 0>{});
    fetch(std::integral_constant<int, 1>{});
    coefs(std::integral_constant<int, 0>{});
    static_for<kT>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s + 1 < kT) coefs(std::integral_constant<int, s + 1>{});
      if constexpr (s + 2 == kT / 2) {
        read_half(st.x + w.c * kXS, xv, kT / 2);
        read_half(st.d + w.c * kXS, dv, kT / 2);
      }
      if constexpr (s + 2 < kT) fetch(std::integral_constant<int, s + 2>{});
      h[0] = __builtin_fmaf(ca[s & 1][0], h[0], cb[s & 1][0]);
      float acc = cc[s & 1][0] * h[0];
#pragma unroll
      for (int n = 1; n < 4; ++n) {
        h[n] = __builtin_fmaf(ca[s & 1][n], h[n], cb[s & 1][n]);
        acc = __builtin_fmaf(cc[s & 1][n], h[n], acc);
      }
      pin(acc);
      p[s & 3] = acc;
      if constexpr ((s & 3) == 3) {
        constexpr int j = s / 4;
        const float S = rows_transpose_sum(tw, w, p[0], p[1], p[2], p[3]);
        const float xe = st.x[w.c * kXS + 4 * j + w.r];
        yv[j] = finish(S, xe, zuse[j]);
      }
    });
    ld.put(rput, sts[cur ^ 1], w, lane);
    Out<IO>::store2(yv[0], yv[1], ry, voff_y, (uint32_t)s0 * row_bytes,
                    (uint32_t)(s0 + 4) * row_bytes);
  };

  if (nfull > 0) {
    RawT ra, rb;
    uint32_t za[2], zb[2];
    ld.issue(ra, 0, lane);
    ld.issue(rb, min(1, nfull - 1) * kT, lane);
    issue_z(za, 0);
    ld.put(ra, sts[0], w, lane);
    int i = 0;
    for (; i + 2 <= nfull; i += 2) {
      tile(i, 0, ra, rb, za, zb);
      tile(i + 1, 1, rb, ra, zb, za);
    }
    if (i < nfull) tile(i, 0, ra, rb, za, zb);
  }

  // ragged end of the chunk (fewer than kT steps): groups of four steps
  // straight from memory; steps past the end contribute a zero partial
  const __amdgpu_buffer_rsrc_t rbb = bc_rsrc(B, k, seqlen);
  const __amdgpu_buffer_rsrc_t rcc = bc_rsrc(C, k, seqlen);
  for (int g0 = nfull * kT; g0 < nsteps; g0 += 4) {
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      p[u] = 0.0f;
      const int s = g0 + u;
      if (s < nsteps) {
        float xs, ds;
        ld.step(s, xs, ds);
        const uint32_t bo = (uint32_t)(s * kDState + n0) * sizeof(IO);
        float acc = 0.0f;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const float Bn = buf<IO>::load(rbb, bo + n * sizeof(IO), 0);
          const float Cn = buf<IO>::load(rcc, bo + n * sizeof(IO), 0);
          float a, b;
          step_coef<V, ZERO_A>(ds, xs, Bn, A2[n], iA[n], a, b);
          h[n] = __builtin_fmaf(a, h[n], b);
          acc = __builtin_fmaf(Cn, h[n], acc);
        }
        p[u] = acc;
      }
    }
    const float S = rows_transpose_sum(tw, w, p[0], p[1], p[2], p[3]);
    if (g0 + w.r < nsteps) {  // this row's step of the group
      const uint32_t so = (uint32_t)g0 * row_bytes;
      const float xs = ld.x_row(g0);
      const float yv = finish(S, xs, HAS_Z ? Raw<IO>::load(rz, ld.voff, so) : 0u);
      Out<IO>::store(yv, ry, voff_y, so);
    }
  }
}

// Chunk pre-pass in the wave-independent form (carry pass 1 beside chunk 0's
// main pass in the first launch): the lane layout and per-wave staging of the
// main pass, without C and the readout.  With no A == 0 in the wave the
// state is carried as g = A*h: g = fma(a, g, fma(a, B*x, -B*x)), converted
// back (h = g/A) at the end of the full tiles.  Sum of delta: row r adds
// steps 2r and 2r + 1 of every tile (fp32 pair, then fp64); the rows' sums
// are added in row order at the end.
template <typename IO, bool ZERO_A, bool FUSED, int V>
__device__ __forceinline__ void chunk_state_w(const IO* __restrict__ x,
                                              const IO* __restrict__ delta,
                                              const IO* __restrict__ B, int64_t seqlen, int dim,
                                              const Chunk& k, const WLane& w,
                                              WStage (&sts)[2], const float (&A2)[4],
                                              const float (&iA)[4], float (&h)[4], double& sd,
                                              const LanePrologue& lp) {
  static_assert((V & kScalarA) == 0, "A per channel uses chunk_state");
  const int lane = threadIdx.x % kWave;
  const int n0 = 4 * w.r;
  using LD = std::conditional_t<FUSED, WFusedLoader<IO, false>, WLoader<IO, false>>;
  using RawT = typename LD::RawTile;
  LD ld;
  ld.init(x, delta, B, B, seqlen, dim, k, w, lp);
  const int nsteps = (int)(k.t_end - k.t_begin);
  const int nfull = nsteps / kT;
  float gs[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) gs[n] = 0.0f;

  auto tile = [&](int tidx, int cur, RawT& rissue, const RawT& rput) {
    ld.issue(rissue, min(tidx + 2, nfull - 1) * kT, lane);
    const WStage& st = sts[cur];
    float xv[kT], dv[kT];
    read_row(st.x + w.c * kXS, xv);
    read_row(st.d + w.c * kXS, dv);
    float bq[2][4];
    auto fetch = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      read_n<4>(st.b + s * kDState + n0, bq[s & 1]);
    };
    float ca[2][4], cb[2][4];
    auto coefs = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        ca[s & 1][n] = fast_exp2(dv[s] * A2[n]);
        pin(ca[s & 1][n]);
      }
      const float dx = dv[s] * xv[s];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const float bx = bq[s & 1][n] * xv[s];
        const float a = ca[s & 1][n];
        if constexpr ((V & kEuler) != 0)
          cb[s & 1][n] = dx * bq[s & 1][n];
        else if constexpr (!ZERO_A)
          cb[s & 1][n] = __builtin_fmaf(a, bx, -bx);  // (a - 1) * B x, for g = A h
        else
          cb[s & 1][n] = (__builtin_isinf(iA[n]) ? dv[s] : (a - 1.0f) * iA[n]) * bx;
        pin(cb[s & 1][n]);
      }
    };
    fetch(std::integral_constant<int, 0>{});
    fetch(std::integral_constant<int, 1>{});
    coefs(std::integral_constant<int, 0>{});
    static_for<kT>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s + 1 < kT) coefs(std::integral_constant<int, s + 1>{});
      if constexpr (s + 2 < kT) fetch(std::integral_constant<int, s + 2>{});
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        gs[n] = __builtin_fmaf(ca[s & 1][n], gs[n], cb[s & 1][n]);
        pin(gs[n]);
      }
    });
    const float2 dd = *reinterpret_cast<const float2*>(st.d + w.c * kXS + 2 * w.r);
    sd += (double)(dd.x + dd.y);
    ld.put(rput, sts[cur ^ 1], w, lane);
  };

  if (nfull > 0) {
    RawT ra, rb;
    ld.issue(ra, 0, lane);
    ld.issue(rb, min(1, nfull - 1) * kT, lane);
    ld.put(ra, sts[0], w, lane);
    int i = 0;
    for (; i + 2 <= nfull; i += 2) {
      tile(i, 0, ra, rb);
      tile(i + 1, 1, rb, ra);
    }
    if (i < nfull) tile(i, 0, ra, rb);
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) h[n] = (ZERO_A || (V & kEuler)) ? gs[n] : gs[n] * iA[n];

  // ragged end of the chunk, one step at a time from memory
  const __amdgpu_buffer_rsrc_t rbb = bc_rsrc(B, k, seqlen);
  for (int s0 = nfull * kT; s0 < nsteps; ++s0) {
    float xs, ds;
    ld.step(s0, xs, ds);
    const uint32_t bo = (uint32_t)(s0 * kDState + n0) * sizeof(IO);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      float a, b;
      step_coef<V, ZERO_A>(ds, xs, buf<IO>::load(rbb, bo + n * sizeof(IO), 0), A2[n], iA[n], a,
                           b);
      h[n] = __builtin_fmaf(a, h[n], b);
    }
    if (w.r == 0) sd += (double)ds;
  }
}

// Pre-pass block (chunk c of one 64-channel group from a zero state) in the
// wave-independent form: writes hloc and the chunk's sum of delta.
template <typename IO, bool FUSED, int V>
__device__ __forceinline__ void pre_block_w(const IO* __restrict__ x, const IO* __restrict__ delta,
                                            const float* __restrict__ A,
                                            const IO* __restrict__ B, float* __restrict__ ws_hloc,
                                            double* __restrict__ ws_sdelta, int64_t seqlen,
                                            int dim, int nchunks, const Chunk& k, WSmem& sm,
                                            const Prologue& pro) {
  const WLane w = wlane(dim);
  WStage(&sts)[2] = sm.st[wave_id()];
  if constexpr (std::is_same<IO, bf16>::value) {
    float4* p = reinterpret_cast<float4*>(&sts[0]);
    constexpr int n = (int)(2 * sizeof(WStage) / sizeof(float4));
    for (int i = threadIdx.x % kWave; i < n; i += kWave) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float A2[4], iA[4], h[4];
  const bool zero = load_A<4, V>(A, w.d, 4 * w.r, A2, iA);
  double sd = 0.0;
  LanePrologue lp{};
  if constexpr (FUSED) lp = lane_prologue(pro, w.d);
  if (__builtin_amdgcn_ballot_w64(zero) != 0)
    chunk_state_w<IO, true, FUSED, V>(x, delta, B, seqlen, dim, k, w, sts, A2, iA, h, sd, lp);
  else
    chunk_state_w<IO, false, FUSED, V>(x, delta, B, seqlen, dim, k, w, sts, A2, iA, h, sd, lp);
  // the rows' sums of delta through the wave's transpose area
  double* td = reinterpret_cast<double*>(sm.tr[wave_id()]);
  asm volatile("" ::: "memory");
  td[w.r * kWCh + w.c] = sd;
  asm volatile("" ::: "memory");
  if (w.active) {
    const size_t cd = ((size_t)k.b * nchunks + k.c) * dim + w.d;
    float* hl = ws_hloc + cd * kDState + 4 * w.r;
#pragma unroll
    for (int j = 0; j < 4; ++j) hl[j] = h[j];
    if (w.r == 0)
      ws_sdelta[cd] = ((td[w.c] + td[kWCh + w.c]) + td[2 * kWCh + w.c]) + td[3 * kWCh + w.c];
  }
}

// The wave-independent form serves plans of 4 waves per group for A per
// (channel, state) with either discretisation rule, with or without the
// fused prologue; A per channel and other plans use scan_chunk and
// chunk_state (with A per channel the wave form measured 9-22% slower).
template <int G, bool FUSED, int V>
constexpr bool kWaveForm = (G == 4 && (V & kScalarA) == 0);

// Main pass of one block in the wave-independent form: `hinit` and `hout`
// point at this lane's 4 states (nullable).
template <typename IO, bool HAS_Z, bool FUSED, int V>
__device__ __forceinline__ void main_block_w(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, const IO* __restrict__ C, const float* __restrict__ Dskip,
    const IO* __restrict__ z, IO* __restrict__ y, const float* hinit, float* hout,
    int64_t seqlen, int dim, const Chunk& k, const WLane& w, WSmem& sm, const Prologue& pro) {
  WStage(&sts)[2] = sm.st[wave_id()];
  float* tw = sm.tr[wave_id()];
  if constexpr (std::is_same<IO, bf16>::value) {
    // bf16 inputs rely on zero lower halves of the slots
    float4* p = reinterpret_cast<float4*>(&sts[0]);
    constexpr int n = (int)(2 * sizeof(WStage) / sizeof(float4));
    for (int i = threadIdx.x % kWave; i < n; i += kWave) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float A2[4], iA[4], h[4];
  const bool zero = load_A<4, V>(A, w.d, 4 * w.r, A2, iA);
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = hinit ? hinit[j] : 0.0f;
  const float Dd = Dskip ? Dskip[w.d] : 0.0f;
  LanePrologue lp{};
  if constexpr (FUSED) lp = lane_prologue(pro, w.d);
  if (__builtin_amdgcn_ballot_w64(zero) != 0)
    scan_chunk_w<IO, HAS_Z, true, FUSED, V>(x, delta, B, C, z, y, Dd, seqlen, dim, k, w, sts, tw,
                                            A2, iA, h, lp);
  else
    scan_chunk_w<IO, HAS_Z, false, FUSED, V>(x, delta, B, C, z, y, Dd, seqlen, dim, k, w, sts,
                                             tw, A2, iA, h, lp);
  if (hout && w.active) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hout[j] = h[j];
  }
}

// Main pass over chunks c_first .. nchunks-1 (grid y: chunk - c_first, grid
// z: batch row).  A chunk c > 0 starts from ws_hin[b, c]; chunk 0 from h0.
// The last chunk writes h_last.
template <typename IO, int G, bool HAS_Z, bool FUSED, int V>
__global__ __launch_bounds__(kWave* G)
__attribute__((amdgpu_waves_per_eu(FUSED ? kFusedWavesPerSimd : kMainWavesPerSimd)))
void scan_fwd_kernel(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, const IO* __restrict__ C, const float* __restrict__ Dskip,
    const IO* __restrict__ z, const float* __restrict__ h0, IO* __restrict__ y,
    float* __restrict__ h_last, const float* __restrict__ ws_hin, int64_t seqlen,
    int64_t chunk_len, int dim, int nchunks, int c_first, Prologue pro) {
  constexpr int NPL = kDState / G;
  const Chunk k = chunk_coords(dim, seqlen, chunk_len, (int)blockIdx.y + c_first, blockIdx.z);
  if constexpr (kWaveForm<G, FUSED, V>) {
    __shared__ WSmem smw;
    const WLane w = wlane(dim);
    const int n0 = 4 * w.r;
    const size_t bd = (size_t)k.b * dim + w.d;
    const float* hinit = nullptr;
    if (k.c > 0)
      hinit = ws_hin + (((size_t)k.b * nchunks + k.c) * dim + w.d) * kDState + n0;
    else if (h0)
      hinit = h0 + bd * kDState + n0;
    float* hout = (k.c == nchunks - 1 && h_last) ? h_last + bd * kDState + n0 : nullptr;
    main_block_w<IO, HAS_Z, FUSED, V>(x, delta, A, B, C, Dskip, z, y, hinit, hout, seqlen, dim, k,
                                      w, smw, pro);
  } else {
    __shared__ MainSmem<G> sm;
    const int n0 = k.g * NPL;
    const size_t bd = (size_t)k.b * dim + k.d;
    const float* hinit = nullptr;
    if (k.c > 0)
      hinit = ws_hin + (((size_t)k.b * nchunks + k.c) * dim + k.d) * kDState + n0;
    else if (h0)
      hinit = h0 + bd * kDState + n0;
    float* hout = (k.c == nchunks - 1 && h_last) ? h_last + bd * kDState + n0 : nullptr;
    main_block<IO, G, HAS_Z, FUSED, V>(x, delta, A, B, C, Dskip, z, y, hinit, hout, seqlen, dim,
                                       k, sm, pro);
  }
}

// ---------------------------------------------------------------------------
// Carry pass 1: end state of every chunk but the last, started from zero,
// plus the chunk's sum of delta.  Same staging as the main kernel, without
// C and the readout.  With no A == 0 in the wave it carries g = A*h.
// ---------------------------------------------------------------------------
template <typename IO, int G, bool ZERO_A, bool FUSED, int V>
__device__ __forceinline__ void chunk_state(const IO* __restrict__ x,
                                            const IO* __restrict__ delta,
                                            const IO* __restrict__ B, int64_t seqlen, int dim,
                                            const Chunk& k, Stage<false>* stages,
                                            const float (&A2)[kDState / G],
                                            const float (&iA)[kDState / G],
                                            float (&h)[kDState / G], double& sd,
                                            const LanePrologue& lp) {
  constexpr int NPL = kDState / G;
  const int lane = k.lane, n0 = k.g * NPL;
  const int nsteps = (int)(k.t_end - k.t_begin);
  const int nfull = nsteps / kT;

  using LD = std::conditional_t<FUSED, FusedLoader<IO, G, false>, Loader<IO, G, false>>;
  using Raw1 = typename LD::RawTile;
  LD ld;
  ld.init(x, delta, B, B, seqlen, dim, k, lp);

  // state carried through the tiles: g = A*h (or h itself when A may be 0)
  float gs[NPL];
#pragma unroll
  for (int n = 0; n < NPL; ++n) gs[n] = 0.0f;

  auto tile = [&](int tidx, int cur, Raw1& rissue, const Raw1& rput) {
    ld.issue(rissue, min(tidx + 2, nfull - 1) * kT, lane);
    const Stage<false>& st = stages[cur];
    float xv[kT], dv[kT];
    read_row(st.x + lane * kXS, xv);
    read_row(st.d + lane * kXS, dv);
    // B of step s is read from LDS two steps before its use; the exp2s and
    // input terms are formed one step before (all exp2s of a step first)
    float bq[2][NPL];
    auto fetch = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      read_n<NPL>(st.b + s * kDState + n0, bq[s & 1]);
    };
    float ca[2][NPL], cb[2][NPL];
    auto coefs = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr ((V & kScalarA) != 0) {
        float a = fast_exp2(dv[s] * A2[0]);
        float c;  // input term / B: (a - 1) x for g = A h (ZOH), delta x (Euler)
        if constexpr ((V & kEuler) != 0)
          c = dv[s] * xv[s];
        else if constexpr (!ZERO_A)
          c = __builtin_fmaf(a, xv[s], -xv[s]);
        else
          c = (__builtin_isinf(iA[0]) ? dv[s] : (a - 1.0f) * iA[0]) * xv[s];
        pin(a);
#pragma unroll
        for (int n = 0; n < NPL; ++n) {
          ca[s & 1][n] = a;
          cb[s & 1][n] = c * bq[s & 1][n];
          pin(cb[s & 1][n]);
        }
      } else {
#pragma unroll
        for (int n = 0; n < NPL; ++n) {
          ca[s & 1][n] = fast_exp2(dv[s] * A2[n]);
          pin(ca[s & 1][n]);
        }
        const float dx = dv[s] * xv[s];
#pragma unroll
        for (int n = 0; n < NPL; ++n) {
          const float bx = bq[s & 1][n] * xv[s];
          const float a = ca[s & 1][n];
          if constexpr ((V & kEuler) != 0)
            cb[s & 1][n] = dx * bq[s & 1][n];
          else if constexpr (!ZERO_A)
            cb[s & 1][n] = __builtin_fmaf(a, bx, -bx);  // (a - 1) * B x, for g = A h
          else
            cb[s & 1][n] = (__builtin_isinf(iA[n]) ? dv[s] : (a - 1.0f) * iA[n]) * bx;
          pin(cb[s & 1][n]);
        }
      }
    };
    fetch(std::integral_constant<int, 0>{});
    fetch(std::integral_constant<int, 1>{});
    coefs(std::integral_constant<int, 0>{});
    static_for<kT>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s + 1 < kT) coefs(std::integral_constant<int, s + 1>{});
      if constexpr (s + 2 < kT) fetch(std::integral_constant<int, s + 2>{});
#pragma unroll
      for (int n = 0; n < NPL; ++n) {
        gs[n] = __builtin_fmaf(ca[s & 1][n], gs[n], cb[s & 1][n]);
        pin(gs[n]);
      }
    });
    // sum of delta over the tile: pairwise in fp32, then into fp64; only
    // wave 0 publishes it, so only wave 0 computes it (a wave-uniform branch)
    if (k.g == 0) {
      float t4[kT / 2];
#pragma unroll
      for (int j = 0; j < kT / 2; ++j) t4[j] = dv[2 * j] + dv[2 * j + 1];
#pragma unroll
      for (int w = kT / 4; w >= 1; w /= 2)
#pragma unroll
        for (int j = 0; j < w; ++j) t4[j] = t4[j] + t4[j + w];
      sd += (double)t4[0];
    }
    ld.put(rput, stages[cur ^ 1], lane);
    __syncthreads();
  };

  if (nfull > 0) {
    Raw1 ra, rb;
    ld.issue(ra, 0, lane);
    ld.issue(rb, min(1, nfull - 1) * kT, lane);
    ld.put(ra, stages[0], lane);
    __syncthreads();
    int i = 0;
    for (; i + 2 <= nfull; i += 2) {
      tile(i, 0, ra, rb);
      tile(i + 1, 1, rb, ra);
    }
    if (i < nfull) tile(i, 0, ra, rb);
  }
#pragma unroll
  for (int n = 0; n < NPL; ++n) h[n] = (ZERO_A || (V & kEuler)) ? gs[n] : gs[n] * iA[n];

  // ragged end of the chunk
  const __amdgpu_buffer_rsrc_t rbb = bc_rsrc(B, k, seqlen);
  for (int s0 = nfull * kT; s0 < nsteps; ++s0) {
    float xs, ds;
    ld.step(s0, xs, ds);
    const uint32_t bo = (uint32_t)(s0 * kDState + n0) * sizeof(IO);
#pragma unroll
    for (int n = 0; n < NPL; ++n) {
      float a, b;
      step_coef<V, ZERO_A>(ds, xs, buf<IO>::load(rbb, bo + n * sizeof(IO), 0), A2[n], iA[n], a,
                           b);
      h[n] = __builtin_fmaf(a, h[n], b);
    }
    sd += (double)ds;
  }
}

// Carry pass 1 of one block: its 64 channels over chunk k from a zero state;
// stores the end state and (wave 0) the chunk's sum of delta.
template <typename IO, int G, bool FUSED, int V>
__device__ __forceinline__ void pre_block(const IO* __restrict__ x, const IO* __restrict__ delta,
                                          const float* __restrict__ A, const IO* __restrict__ B,
                                          float* __restrict__ ws_hloc,
                                          double* __restrict__ ws_sdelta, int64_t seqlen,
                                          int dim, int nchunks, const Chunk& k,
                                          Stage<false>* stages, const Prologue& pro) {
  constexpr int NPL = kDState / G;
  const int n0 = k.g * NPL;
  clear_stages<IO, false>(stages, kWave * G);
  float A2[NPL], iA[NPL], h[NPL];
  const bool zero = load_A<NPL, V>(A, k.d, n0, A2, iA);
  double sd = 0.0;
  LanePrologue lp{};
  if constexpr (FUSED) lp = lane_prologue(pro, k.d);
  __syncthreads();  // stages cleared
  if (__builtin_amdgcn_ballot_w64(zero) != 0)
    chunk_state<IO, G, true, FUSED, V>(x, delta, B, seqlen, dim, k, stages, A2, iA, h, sd, lp);
  else
    chunk_state<IO, G, false, FUSED, V>(x, delta, B, seqlen, dim, k, stages, A2, iA, h, sd, lp);
  if (k.active) {
    const size_t cd = ((size_t)k.b * nchunks + k.c) * dim + k.d;
    float* hl = ws_hloc + cd * kDState + n0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) hl[j] = h[j];
    if (k.g == 0) ws_sdelta[cd] = sd;
  }
}

// Carry pass 1 of the three-pass schedule: chunks 0 .. nchunks-2 (grid y),
// each from a zero state.
template <typename IO, int G, bool FUSED, int V>
__global__ __launch_bounds__(kWave* G) __attribute__((amdgpu_waves_per_eu(kCarryWavesPerSimd)))
void scan_chunk_state_kernel(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, float* __restrict__ ws_hloc, double* __restrict__ ws_sdelta,
    int64_t seqlen, int64_t chunk_len, int dim, int nchunks, Prologue pro) {
  __shared__ Stage<false> stages[2];
  const Chunk k = chunk_coords(dim, seqlen, chunk_len, blockIdx.y, blockIdx.z);
  pre_block<IO, G, FUSED, V>(x, delta, A, B, ws_hloc, ws_sdelta, seqlen, dim, nchunks, k, stages,
                             pro);
}

// First launch of the two-launch schedule (grid x: channel group, y: batch
// row, z: role).  Chunk 0 needs no carry, so its main pass runs here at once
// (z == 0): it writes y of chunk 0 and the state entering chunk 1 into
// ws_hin.  The other blocks (z = c in 1 .. nchunks-2) run chunk c from a zero
// state, as carry pass 1 does.  The blocks of chunk 0 come first in dispatch
// order; they are the longest.  Chunk 0's own pre-pass, which the three-pass
// schedule spends, is never needed.
template <typename IO, int G, bool HAS_Z, bool FUSED, int V>
__global__ __launch_bounds__(kWave* G)
__attribute__((amdgpu_waves_per_eu(FUSED ? kFusedWavesPerSimd : kMainWavesPerSimd)))
void scan_first_kernel(
    const IO* __restrict__ x, const IO* __restrict__ delta, const float* __restrict__ A,
    const IO* __restrict__ B, const IO* __restrict__ C, const float* __restrict__ Dskip,
    const IO* __restrict__ z, const float* __restrict__ h0, IO* __restrict__ y,
    float* __restrict__ ws_hloc, double* __restrict__ ws_sdelta, float* __restrict__ ws_hin,
    int64_t seqlen, int64_t chunk_len, int dim, int nchunks, Prologue pro) {
  constexpr int NPL = kDState / G;
  using MainS = std::conditional_t<kWaveForm<G, FUSED, V>, WSmem, MainSmem<G>>;
  __shared__ union {
    MainS main;
    Stage<false> pre[2];
  } sm;
  const Chunk k = chunk_coords(dim, seqlen, chunk_len, blockIdx.z, blockIdx.y);
  if (k.c == 0) {
    if constexpr (kWaveForm<G, FUSED, V>) {
      const WLane w = wlane(dim);
      const int n0 = 4 * w.r;
      const size_t bd = (size_t)k.b * dim + w.d;
      const float* hinit = h0 ? h0 + bd * kDState + n0 : nullptr;
      float* hout = ws_hin + (((size_t)k.b * nchunks + 1) * dim + w.d) * kDState + n0;
      main_block_w<IO, HAS_Z, FUSED, V>(x, delta, A, B, C, Dskip, z, y, hinit, hout, seqlen, dim,
                                        k, w, sm.main, pro);
    } else {
      const int n0 = k.g * NPL;
      const size_t bd = (size_t)k.b * dim + k.d;
      const float* hinit = h0 ? h0 + bd * kDState + n0 : nullptr;
      float* hout = ws_hin + (((size_t)k.b * nchunks + 1) * dim + k.d) * kDState + n0;
      main_block<IO, G, HAS_Z, FUSED, V>(x, delta, A, B, C, Dskip, z, y, hinit, hout, seqlen,
                                         dim, k, sm.main, pro);
    }
  } else {
    if constexpr (kWaveForm<G, FUSED, V>)
      pre_block_w<IO, FUSED, V>(x, delta, A, B, ws_hloc, ws_sdelta, seqlen, dim, nchunks, k, sm.main,
                                  pro);
    else
      pre_block<IO, G, FUSED, V>(x, delta, A, B, ws_hloc, ws_sdelta, seqlen, dim, nchunks, k,
                                 sm.pre, pro);
  }
}

// ---------------------------------------------------------------------------
// Carry pass 2: the state entering every chunk.  Chunk c maps its entering
// state h to P_c h + hloc_c with P_c = exp(A * sum of delta over chunk c) (the
// product of the chunk's Abar as one exponential); applying the maps in
// order from h0 gives every chunk's entering state (paperlens tutorial,
// parallel-scan section: the update composes associatively).  One thread per
// (b, d, n) walks the chunks in order; consecutive threads take consecutive
// (d, n), so every load and store of a step is one coalesced row, and the
// loads of four steps are issued before their updates.
//
// In the two-launch schedule the first launch already gives the state
// entering chunk 1 (chunk 0's main pass ends there), so the walk starts at
// chunk c_first = 1.
//
// With `reverse` set the same composition runs from the last chunk to the
// first (chunk c is addressed as nchunks - 1 - c): the backward pass uses it
// for the adjoint of the state, which flows from the end of the sequence to
// its start with the same per-chunk decay.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scan_carry_kernel(
    const float* __restrict__ A, const float* __restrict__ h0,
    const float* __restrict__ ws_hloc, const double* __restrict__ ws_sdelta,
    float* __restrict__ ws_hin, int batch, int dim, int nchunks, int a_scalar, int reverse,
    int c_first) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)batch * dim * kDState;
  if (gid >= total) return;
  const int n = (int)(gid % kDState);
  const int64_t bd = gid / kDState;
  const int d = (int)(bd % dim);
  const int64_t b = bd / dim;
  const double A2 = (double)(A[a_scalar ? (size_t)d : (size_t)d * kDState + n] * kLog2e);
  auto cd = [&](int c) {
    return ((size_t)b * nchunks + (reverse ? nchunks - 1 - c : c)) * dim + d;
  };
  // c_first == 0: from h0 (or zero), which is the state entering chunk 0;
  // c_first > 0: from the state entering chunk c_first, already in ws_hin
  float h;
  if (c_first == 0) {
    h = h0 ? h0[gid] : 0.0f;
    ws_hin[cd(0) * kDState + n] = h;
  } else {
    h = ws_hin[cd(c_first) * kDState + n];
  }
  constexpr int U = 4;
  int c = c_first;
  for (; c + U <= nchunks - 1; c += U) {
    float P[U], H[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      P[u] = fast_exp2((float)(A2 * ws_sdelta[cd(c + u)]));
      H[u] = ws_hloc[cd(c + u) * kDState + n];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      h = __builtin_fmaf(P[u], h, H[u]);
      ws_hin[cd(c + u + 1) * kDState + n] = h;
    }
  }
  for (; c < nchunks - 1; ++c) {
    h = __builtin_fmaf(fast_exp2((float)(A2 * ws_sdelta[cd(c)])), h, ws_hloc[cd(c) * kDState + n]);
    ws_hin[cd(c + 1) * kDState + n] = h;
  }
}

__global__ __launch_bounds__(256) void copy_state_kernel(const float* __restrict__ h0,
                                                         float* __restrict__ h_last,
                                                         int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) h_last[i] = h0 ? h0[i] : 0.0f;
}

template <typename IO, int G, bool FUSED, int V>
hipError_t launch_scan_t(const ScanArgs& a, int phase, hipStream_t stream) {
  const IO* x = static_cast<const IO*>(a.x);
  const IO* delta = static_cast<const IO*>(a.delta);
  const IO* B = static_cast<const IO*>(a.B);
  const IO* C = static_cast<const IO*>(a.C);
  const IO* z = static_cast<const IO*>(a.z);
  IO* y = static_cast<IO*>(a.y);
  const unsigned gx = (unsigned)((a.dim + kWave - 1) / kWave);
  const int64_t threads = (int64_t)a.batch * a.dim * kDState;
  const dim3 carry_grid((unsigned)((threads + 255) / 256));
  const int vs = (V & kScalarA) ? 1 : 0;
  hipError_t e;
  if ((phase & kPhaseThreePass) || a.nchunks <= 1) {
    // three-pass schedule: carry pass 1 on chunks 0 .. K-2, carry pass 2 from
    // h0, main pass on every chunk (also the one-chunk case: main pass only)
    if (a.nchunks > 1 && (phase & 1)) {
      // the carry pass has no readout to share, so it splits the states over
      // more waves (two per wave) for latency hiding
      constexpr int GC = G < 8 ? 8 : G;
      dim3 grid1(gx, (unsigned)(a.nchunks - 1), (unsigned)a.batch);
      hipLaunchKernelGGL((scan_chunk_state_kernel<IO, GC, FUSED, V>), grid1, dim3(kWave * GC), 0,
                         stream, x, delta, a.A, B, a.ws_hloc, a.ws_sdelta, a.seqlen, a.chunk_len,
                         a.dim, a.nchunks, a.pro);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(scan_carry_kernel, carry_grid, dim3(256), 0, stream, a.A, a.h0,
                         a.ws_hloc, a.ws_sdelta, a.ws_hin, a.batch, a.dim, a.nchunks, vs, 0, 0);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (!(phase & 2)) return hipSuccess;
    dim3 grid(gx, (unsigned)a.nchunks, (unsigned)a.batch);
    if (a.z)
      hipLaunchKernelGGL((scan_fwd_kernel<IO, G, true, FUSED, V>), grid, dim3(kWave * G), 0,
                         stream, x, delta, a.A, B, C, a.Dskip, z, a.h0, y, a.h_last, a.ws_hin,
                         a.seqlen, a.chunk_len, a.dim, a.nchunks, 0, a.pro);
    else
      hipLaunchKernelGGL((scan_fwd_kernel<IO, G, false, FUSED, V>), grid, dim3(kWave * G), 0,
                         stream, x, delta, a.A, B, C, a.Dskip, static_cast<const IO*>(nullptr),
                         a.h0, y, a.h_last, a.ws_hin, a.seqlen, a.chunk_len, a.dim, a.nchunks, 0,
                         a.pro);
    return hipGetLastError();
  }
  // two-launch schedule (K >= 2): the first launch runs chunk 0's main pass
  // beside carry pass 1 of chunks 1 .. K-2; carry pass 2 composes from the
  // state entering chunk 1; the second launch is the main pass of chunks
  // 1 .. K-1
  if (phase & 1) {
    dim3 grid1(gx, (unsigned)a.batch, (unsigned)(a.nchunks - 1));
    if (a.z)
      hipLaunchKernelGGL((scan_first_kernel<IO, G, true, FUSED, V>), grid1, dim3(kWave * G), 0,
                         stream, x, delta, a.A, B, C, a.Dskip, z, a.h0, y, a.ws_hloc,
                         a.ws_sdelta, a.ws_hin, a.seqlen, a.chunk_len, a.dim, a.nchunks, a.pro);
    else
      hipLaunchKernelGGL((scan_first_kernel<IO, G, false, FUSED, V>), grid1, dim3(kWave * G), 0,
                         stream, x, delta, a.A, B, C, a.Dskip, static_cast<const IO*>(nullptr),
                         a.h0, y, a.ws_hloc, a.ws_sdelta, a.ws_hin, a.seqlen, a.chunk_len, a.dim,
                         a.nchunks, a.pro);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.nchunks > 2) {
      hipLaunchKernelGGL(scan_carry_kernel, carry_grid, dim3(256), 0, stream, a.A, a.h0,
                         a.ws_hloc, a.ws_sdelta, a.ws_hin, a.batch, a.dim, a.nchunks, vs, 0, 1);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (!(phase & 2)) return hipSuccess;
  dim3 grid(gx, (unsigned)(a.nchunks - 1), (unsigned)a.batch);
  if (a.z)
    hipLaunchKernelGGL((scan_fwd_kernel<IO, G, true, FUSED, V>), grid, dim3(kWave * G), 0, stream,
                       x, delta, a.A, B, C, a.Dskip, z, a.h0, y, a.h_last, a.ws_hin, a.seqlen,
                       a.chunk_len, a.dim, a.nchunks, 1, a.pro);
  else
    hipLaunchKernelGGL((scan_fwd_kernel<IO, G, false, FUSED, V>), grid, dim3(kWave * G), 0, stream,
                       x, delta, a.A, B, C, a.Dskip, static_cast<const IO*>(nullptr), a.h0, y,
                       a.h_last, a.ws_hin, a.seqlen, a.chunk_len, a.dim, a.nchunks, 1, a.pro);
  return hipGetLastError();
}

template <typename IO, int V>
hipError_t launch_variant(const ScanArgs& a, int G, int phase, hipStream_t stream) {
  switch (G) {  // the variants have kernels for 2, 4 and 8 waves per group
    case 2: return launch_scan_t<IO, 2, false, V>(a, phase, stream);
    case 4: return launch_scan_t<IO, 4, false, V>(a, phase, stream);
    case 8: return launch_scan_t<IO, 8, false, V>(a, phase, stream);
  }
  return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_scan_io(const ScanArgs& a, int G, int phase, hipStream_t stream) {
  const int V = (a.a_per_channel ? kScalarA : 0) | (a.euler ? kEuler : 0);
  if (a.pro.d_conv > 0) {
    if (V != 0) return hipErrorInvalidValue;
    switch (G) {  // the fused loader needs G <= kT
      case 2: return launch_scan_t<IO, 2, true, 0>(a, phase, stream);
      case 4: return launch_scan_t<IO, 4, true, 0>(a, phase, stream);
      case 8: return launch_scan_t<IO, 8, true, 0>(a, phase, stream);
    }
    return hipErrorInvalidValue;
  }
  switch (V) {
    case kScalarA: return launch_variant<IO, kScalarA>(a, G, phase, stream);
    case kEuler: return launch_variant<IO, kEuler>(a, G, phase, stream);
    case kScalarA | kEuler: return launch_variant<IO, kScalarA | kEuler>(a, G, phase, stream);
  }
  switch (G) {
    case 2: return launch_scan_t<IO, 2, false, 0>(a, phase, stream);
    case 4: return launch_scan_t<IO, 4, false, 0>(a, phase, stream);
    case 8: return launch_scan_t<IO, 8, false, 0>(a, phase, stream);
    case 16: return launch_scan_t<IO, 16, false, 0>(a, phase, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int scan_tile_steps() { return kChunkAlign; }

hipError_t launch_carry(const float* A, int a_per_channel, const float* init,
                        const float* ws_loc, const double* ws_sdelta, float* ws_in, int batch,
                        int dim, int nchunks, bool reverse, hipStream_t stream) {
  if (nchunks <= 1) return hipSuccess;
  const int64_t threads = (int64_t)batch * dim * kDState;
  hipLaunchKernelGGL(scan_carry_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, A, init, ws_loc, ws_sdelta, ws_in, batch, dim, nchunks,
                     a_per_channel, reverse ? 1 : 0, 0);
  return hipGetLastError();
}

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
