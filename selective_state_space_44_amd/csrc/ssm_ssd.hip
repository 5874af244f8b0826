// ssm_ssd.hip -- the selective scan with a step size and a decay rate shared
// by each head of 64 channels, computed in its masked-matrix form on the
// matrix cores (gfx950 bf16 MFMA, fp32 accumulation).
//
// Method (ihouse article on Mamba-3, section on Mamba's evolution: with A
// reduced to a scalar the bulk of the SSM's work becomes masked matrix
// products; paperlens tutorial, section on the parallel scan: the recurrence
// composes chunk by chunk).  For one batch row, head h (decay rate a, step
// dt_t) and a chunk of Q = 32 steps, with s_t = a * sum_{r<=t} dt_r inside
// the chunk and coef_t the input coefficient of step t ((exp(a dt_t) - 1)/a
// for the zero-order hold, dt_t for the Euler rule, dt_t at a = 0):
//
//   y_i   = sum_{j<=i} M_ij exp(s_i - s_j) coef_j x_j  +  exp(s_i) C_i . h_in
//   h_out = exp(s_last) h_in + sum_j exp(s_last - s_j) coef_j x_j B_j^T
//
// with M = C B^T (Q x Q, contraction over the N states), then
// y = (y + D x) * SiLU(z).  Four products per chunk: M (the same for every
// head of a batch row), P X with P = M masked to j <= i and weighted
// (contraction over the steps), C h_in^T (over the states) and B^T (w x) with
// w_t = exp(s_last - s_t) coef_t (over the steps).
//
// Two kernels:
//  * ssd_prep_kernel, one block per (batch row, chunk), writes what every
//    head of the row reads: the three lower-triangular 16 x 16 tiles of M,
//    B^T (states as rows, the chunk's steps contiguous) and C with its states
//    in the order the C h_in product takes them.
//  * ssd_scan_kernel, one block per (half head of 32 channels, batch row),
//    walks the chunks in order, so the state never leaves the registers.
//    Its 4 waves are 2 channel tiles x 2 state halves: wave (pt, nh) holds
//    h[n][p] for 16 channels and N/2 states as MFMA accumulator tiles.
//
// One barrier per chunk.  Phase A: waves 0..2 build one tile of P each from
// M, wave 3 the next chunk's per-step values (decay exponents, coefficients,
// weights); every wave computes C h_in over its state half for the chunk's
// two 16-step row tiles, keeps row tile nh and passes the other to the wave
// holding the other state half of the same channels.  Barrier.  Phase B:
// each wave finishes its row tile (P X, the two halves of C h_in, skip,
// gate, store) and updates its part of the state.  C, B^T and x of a chunk
// are copied into LDS by the buffer unit (buffer_load ... lds, 1 KB per wave
// and transfer) one chunk ahead, double-buffered; P and the partial sums are
// double-buffered and the per-step values triple-buffered, so a wave can run
// the next chunk's phase A while others still finish phase B.  In LDS the
// 16-byte pieces of each row are permuted by a function of the row, so that
// the operand reads of 16 consecutive rows fall on distinct banks.
//
// Precision: B, C and x are bf16 inputs, exact as MFMA operands.  The other
// operands -- the masked weights P, the state h and the weighted inputs w x --
// are fp32 values; each is split into a bf16 high part and a bf16 low part
// (v = hi + lo to about 2^-17 |v|) and both parts are multiplied, so every
// product carries ~16 significant bits and all sums are fp32.  The state
// stays fp32 between chunks.
//
// MFMA lane layouts (v_mfma_f32_16x16x32_bf16 only; 16 x 16 tiles, lane l,
// g = l / 16):
//   A operand: row l % 16, k slots 8g..8g+7
//   B operand: column l % 16, the same k slots
//   result:    column l % 16, rows 4g..4g+3
// A product pairs the k slots of A and B one to one, so any permutation of
// the contraction index applied to both operands gives the same sum.  The
// kernels use that freedom so that result tiles become the next product's
// operand without a trip through LDS: slots 0..3 of lane group g hold
// contraction indices 4g..4g+3 of a 32-wide step and slots 4..7 the indices
// 16+4g..16+4g+3 (the rows of two result tiles).  B^T and C in the workspace
// are stored in that order.  The 16x16x16 form is not used: in one compiled
// schedule the result rows 0-1 of such a product were read before it had
// completed.

#include <type_traits>

#include "ssm_device.h"
#include "ssm_launch.h"
#include "ssm_mfma.h"

namespace ssm {
namespace {

constexpr int kQ = kSsdChunk;     // steps per chunk (32)
constexpr int kHD = 64;           // channels per head
constexpr int kBC = 32;           // channels per block (half a head)
constexpr int kSsdThreads = 256;  // 4 waves: 2 channel tiles x 2 state halves
constexpr int kTiles = 3;         // lower-triangular tiles (0,0), (1,0), (1,1)

// s_waitcnt immediate: at most n (< 16) vector memory operations in flight,
// LDS and export counters not waited for.
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15); }

// Slot of 16-byte piece p in a 64-byte LDS row r is p ^ swz4(r): for any 8
// (and any 16) consecutive rows and a fixed p the slots fall on distinct
// banks.
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Inclusive prefix sum of v over lanes 0..31 (lanes 32..63 get that of
// 32..63): shifts by 1, 2, 4, 8 within rows of 16 lanes, then row 0's total
// added to row 1 (DPP row broadcast), with no trip through LDS.
__device__ __forceinline__ float prefix32(float v) {
  auto add = [](float x, int t) { return x + __int_as_float(t); };
  float s = v;
  s = add(s, __builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x111, 0xf, 0xf, false));  // row_shr:1
  s = add(s, __builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x112, 0xf, 0xf, false));  // row_shr:2
  s = add(s, __builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x114, 0xf, 0xf, false));  // row_shr:4
  s = add(s, __builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x118, 0xf, 0xf, false));  // row_shr:8
  return add(s, __builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x142, 0xa, 0xf, false));  // row_bcast:15
}

// Input coefficient of the zero-order hold, (exp(dt a) - 1) / a = dt phi(u)
// with u = dt a and phi(u) = (exp(u) - 1) / u: for |u| <= 1/2 the Taylor
// series of phi to u^7 (truncation below 2e-8 relative), else the hardware
// exp2 (the difference exp(u) - 1 then loses at most a factor 1.6 of its
// relative accuracy) times 1 / a.
__device__ __forceinline__ float zoh_coef(float dt, float a, float inv_a) {
  const float u = dt * a;
  float ph = 1.0f / 40320.0f;
  ph = __builtin_fmaf(ph, u, 1.0f / 5040.0f);
  ph = __builtin_fmaf(ph, u, 1.0f / 720.0f);
  ph = __builtin_fmaf(ph, u, 1.0f / 120.0f);
  ph = __builtin_fmaf(ph, u, 1.0f / 24.0f);
  ph = __builtin_fmaf(ph, u, 1.0f / 6.0f);
  ph = __builtin_fmaf(ph, u, 0.5f);
  ph = __builtin_fmaf(ph, u, 1.0f);
  const float big = (fast_exp2(u * kLog2e) - 1.0f) * inv_a;
  return __builtin_fabsf(u) <= 0.5f ? dt * ph : big;
}

template <int N>
struct SsdSmem {
  // C of a chunk (rows of N states in the workspace order); piece p of row t
  // at slot p ^ (t & (N / 8 - 1))
  alignas(16) uint16_t cs[2][kQ * N];
  // B^T of a chunk (rows of 32 steps); piece p of row n at slot p ^ swz4(n)
  alignas(16) uint16_t bts[2][N * kQ];
  // x of the block's 32 channels (rows of 64 bytes); slot p ^ swz4(t)
  alignas(16) uint16_t xs[2][kQ * kBC];
  // masked weights per tile and lane, bf16 high and low parts of q = 0..3
  alignas(16) u32x2_t pmh[2][kTiles][kWave];
  alignas(16) u32x2_t pml[2][kTiles][kWave];
  // C h_in over one state half for the other half's wave:
  // [channel tile][row tile][lane]
  alignas(16) f32x4_t part[2][2][2][kWave];
  // per-step values: s_t log2(e), coef_t, w_t, exp(s_t)
  alignas(16) float ps[4][4][kQ];
};

// ---------------------------------------------------------------------------
// Per (batch row, chunk) operands shared by every head, into the workspace:
//   ws_mt: [batch][nck][3][64 lanes] f32x4, lane (r, g) of tile (I, J)
//          holding M[16 I + r][16 J + 4 g + q], q = 0..3
//   ws_bt: [batch][nck][N][32] bf16, row n holding B[t][n] with step 4g+s at
//          position 8g + s and step 16+4g+s at 8g + 4 + s (s < 4)
//   ws_cp: [batch][nck][32][N] bf16, row t holding C[t][n] with state
//          32k+4g+s at position 32k + 8g + s and 32k+16+4g+s at 32k+8g+4+s
// Steps past the end of the sequence are zero.
template <int N>
__global__ __launch_bounds__(256) void ssd_prep_kernel(SsdArgs a) {
  constexpr int kRow = N + 8;  // bf16 per staged row (16-byte pad: distinct banks)
  __shared__ __align__(16) uint16_t bs[kQ][kRow];
  __shared__ __align__(16) uint16_t cs[kQ][kRow];
  const int64_t c = blockIdx.x;
  const int64_t b = (int64_t)blockIdx.y + a.row0;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t L = a.seqlen, t0 = c * kQ;
  const uint32_t rows = (uint32_t)(L - t0 < kQ ? L - t0 : (int64_t)kQ);
  const __amdgpu_buffer_rsrc_t rsb =
      make_rsrc(static_cast<const uint16_t*>(a.B) + (b * L + t0) * N, rows * N * 2u);
  const __amdgpu_buffer_rsrc_t rsc =
      make_rsrc(static_cast<const uint16_t*>(a.C) + (b * L + t0) * N, rows * N * 2u);
  constexpr int kPer = N / 8;  // 16-byte pieces per row
  for (int i = tid; i < kQ * kPer; i += 256) {
    const int t = i / kPer, col = (i % kPer) * 8;
    const uint32_t off = (uint32_t)(t * N + col) * 2u;
    *reinterpret_cast<u32x4_t*>(&bs[t][col]) =
        __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsb, off, 0, 0));
    *reinterpret_cast<u32x4_t*>(&cs[t][col]) =
        __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsc, off, 0, 0));
  }
  __syncthreads();

  const size_t chunk = (size_t)b * a.nck + c;
  // M^T tiles: A operand B rows (j), B operand C rows (i) -> m[q] = C_i . B_j
  // with i = 16 I + r16 (the lane's column), j = 16 J + 4 g + q
  if (w < kTiles) {
    const int I = w > 0 ? 1 : 0, J = w == 1 ? 0 : I;
    f32x4_t m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < N / 32; ++k)
      m = mfma_k32(lds128(&bs[16 * J + r16][32 * k + 8 * g]),
                   lds128(&cs[16 * I + r16][32 * k + 8 * g]), m);
    reinterpret_cast<f32x4_t*>(a.ws_mt)[(chunk * kTiles + w) * kWave + lane] = m;
  }
  // B^T: 16-byte piece gg of row n
  uint16_t* bt = static_cast<uint16_t*>(a.ws_bt) + chunk * N * kQ;
  for (int i = tid; i < N * 4; i += 256) {
    const int n = i >> 2, gg = i & 3;
    const int tlo = 4 * gg, thi = tlo + 16;
    const u32x4_t v = {bs[tlo][n] | ((uint32_t)bs[tlo + 1][n] << 16),
                       bs[tlo + 2][n] | ((uint32_t)bs[tlo + 3][n] << 16),
                       bs[thi][n] | ((uint32_t)bs[thi + 1][n] << 16),
                       bs[thi + 2][n] | ((uint32_t)bs[thi + 3][n] << 16)};
    *reinterpret_cast<u32x4_t*>(bt + (size_t)n * kQ + 8 * gg) = v;
  }
  // C reordered: 16-byte piece pc of row t
  uint16_t* cp = static_cast<uint16_t*>(a.ws_cp) + chunk * kQ * N;
  for (int i = tid; i < kQ * kPer; i += 256) {
    const int t = i / kPer, pc = i % kPer;
    const int lo = 32 * (pc >> 2) + 4 * (pc & 3);
    *reinterpret_cast<u32x4_t*>(cp + (size_t)t * N + 8 * pc) =
        cat(lds64(&cs[t][lo]), lds64(&cs[t][lo + 16]));
  }
}

// ---------------------------------------------------------------------------
// The chunk walk.  PRE: the state-only pass over segments 0..nseg-2 (no
// outputs): end state from zero and the log2 of the segment's decay, into
// the workspace.
template <int N, bool HAS_Z, bool EULER, bool PRE>
__global__ __launch_bounds__(kSsdThreads) __attribute__((amdgpu_waves_per_eu(3)))
void ssd_scan_kernel(SsdArgs a) {
  constexpr int NT2 = N / 32;   // 16-state tiles per wave (its half of the N)
  constexpr int NK = N / 64;    // 32-state contraction steps per state half
  constexpr int CPW = N / 64;   // 1 KB transfers per wave for C and for B^T
  extern __shared__ __align__(16) unsigned char ssd_smem_raw[];
  SsdSmem<N>& sm = *reinterpret_cast<SsdSmem<N>*>(ssd_smem_raw);

  const int H = a.nheads;
  // Block -> (head, half): the two halves of a head get block ids 8 apart,
  // so that they run on the same XCD (blocks are dealt to the 8 XCDs in turn)
  // and share its L2 for the 128-byte rows of x and z they split.
  int h, half;
  {
    const int i = blockIdx.x, grp = i >> 4, r = i & 15;
    if (8 * grp + 8 <= H) {
      h = 8 * grp + (r & 7);
      half = r >> 3;
    } else {  // last, partial group of heads: plain order
      h = 8 * grp + (r >> 1);
      half = r & 1;
    }
  }
  const int64_t b = (int64_t)blockIdx.y + a.row0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = wave_id();
  const int r16 = lane & 15, g = lane >> 4;
  const int pt = w & 1, nh = w >> 1;  // channel tile, state half (= own row tile)
  const int dim = a.dim;
  const int64_t L = a.seqlen;
  const float Ah = a.A[h];
  const float A2 = Ah * kLog2e;
  const bool coef_is_dt = EULER || Ah == 0.0f;  // the Euler rule, or the hold's a -> 0 limit
  const int cb = h * kHD + kBC * half;          // first channel of the block
  const int p = 16 * pt + r16;                  // this lane's channel in the block
  const int d = cb + p;
  const float Dp = a.Dskip ? a.Dskip[d] : 0.0f;
  // this block's steps [tb, te), its first chunk gc0 of the workspace
  const int seg = blockIdx.z;
  const int64_t tb = (int64_t)seg * a.seg_len;
  const int64_t te = tb + a.seg_len < L ? tb + a.seg_len : L;
  const int64_t gc0 = tb / kQ;
  const int64_t nck = (te - tb + kQ - 1) / kQ;
  const size_t seg_row = (size_t)b * a.nseg + seg;  // (batch row, segment) of the workspace
  const size_t soff = 16 * nh * NT2 + 4 * g;        // this lane's first state

  // state tile j: st[j][q] = h[n = 16 (nh NT2 + j) + 4 g + q][p]
  f32x4_t st[NT2];
  {
    const float* src = nullptr;
    if (!PRE) {
      if (seg > 0)
        src = a.ws_hin + (seg_row * dim + d) * N + soff;
      else if (a.h0)
        src = a.h0 + ((size_t)b * dim + d) * N + soff;
    }
#pragma unroll
    for (int j = 0; j < NT2; ++j)
      st[j] = src ? *reinterpret_cast<const f32x4_t*>(src + 16 * j) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float dlog = 0.0f;  // PRE: log2 of the segment's decay

  const u32x4_t ipick = identity_pick(16 * pt, r16, g);
  const u32x4_t ipick4 = identity_pick4(r16, g);
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  // valid steps of the segment's chunk k (none past the end: such loads read
  // zeros); every chunk but the last is full
  const int nck_i = (int)nck;
  const int tail = (int)(te - tb - (int64_t)(nck_i - 1) * kQ);
  auto rows_of = [&](int k) { return (uint32_t)(k < nck_i - 1 ? kQ : k == nck_i - 1 ? tail : 0); };
  // Per-chunk base pointers, advanced by one chunk per iteration (scalar
  // adds instead of 64-bit index arithmetic).
  const size_t row0 = (size_t)b * L + tb;  // first step of the segment
  const uint16_t* xp = static_cast<const uint16_t*>(a.x) + row0 * dim;
  const uint16_t* zp = static_cast<const uint16_t*>(a.z) + row0 * dim;
  uint16_t* yp = static_cast<uint16_t*>(a.y) + row0 * dim;
  const uint16_t* dtp = static_cast<const uint16_t*>(a.dt) + row0 * H;
  const size_t ck0 = (size_t)b * a.nck + gc0;  // first workspace chunk
  const uint16_t* cpp = static_cast<const uint16_t*>(a.ws_cp) + ck0 * kQ * N;
  const uint16_t* btp = static_cast<const uint16_t*>(a.ws_bt) + ck0 * N * kQ;
  const float* mtp = a.ws_mt + ck0 * kTiles * kWave * 4;
  const size_t xstep = (size_t)kQ * dim, dtstep = (size_t)kQ * H;
  constexpr int kCk = kQ * N;                    // elements of a chunk of C or B^T
  constexpr int kMk = kTiles * kWave * 4;        // floats of a chunk of M tiles

  // ---- copies into LDS ------------------------------------------------------
  // Transfer i of wave w fills LDS bytes [1024 (CPW w + i), + 1024) of a
  // buffer; lane l the 16 bytes at 16 l of that.  The source piece of each
  // slot follows the row permutation of the buffer.
  // C of a chunk (workspace pointer) into buffer `buf`
  auto copy_c = [&](int buf, const uint16_t* cpc) {
    if constexpr (!PRE) {
      const __amdgpu_buffer_rsrc_t rsc = make_rsrc(cpc, (uint32_t)(kCk * 2));
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const int pos = 1024 * (CPW * w + i) + 16 * lane;  // byte position in the buffer
        const int t = pos / (2 * N), slot = (pos >> 4) & (N / 8 - 1);
        const int pc = slot ^ (t & (N / 8 - 1));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsc, (__attribute__((address_space(3))) void*)&sm.cs[buf][512 * (CPW * w + i)], 16,
            (uint32_t)(t * N + 8 * pc) * 2u, 0, 0, 0);
      }
    }
  };
  // B^T of a chunk (workspace pointer) into buffer `buf`
  auto copy_bt = [&](int buf, const uint16_t* btc) {
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(btc, (uint32_t)(kCk * 2));
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int pos = 1024 * (CPW * w + i) + 16 * lane;
      const int n = pos >> 6, pc = ((pos >> 4) & 3) ^ swz4(n);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsb, (__attribute__((address_space(3))) void*)&sm.bts[buf][512 * (CPW * w + i)], 16,
          (uint32_t)(n * kQ + 8 * pc) * 2u, 0, 0, 0);
    }
  };
  // x of a chunk (pointer, valid rows) into buffer `buf` (waves 0 and 1,
  // 1 KB each)
  auto copy_x = [&](int buf, const uint16_t* xc, uint32_t rows) {
    if (w < 2) {
      const __amdgpu_buffer_rsrc_t rsx = make_rsrc(xc, rows * (uint32_t)dim * 2u);
      const int t = 16 * w + (lane >> 2), pc = (lane & 3) ^ swz4(t);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsx, (__attribute__((address_space(3))) void*)&sm.xs[buf][512 * w], 16,
          (uint32_t)(t * dim + cb + 8 * pc) * 2u, 0, 0, 0);
    }
  };

  // ---- register loads -------------------------------------------------------
  // M tile w (waves 0..2) of a chunk
  auto load_m = [&](const float* mtc) {
    if (w >= kTiles) return f32x4_t{0.f, 0.f, 0.f, 0.f};
    const __amdgpu_buffer_rsrc_t rsm = make_rsrc(mtc, (uint32_t)(kMk * 4));
    return __builtin_bit_cast(
        f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsm, (uint32_t)lane * 16u, w * kWave * 16, 0));
  };
  // z of row tile nh as the identity A operand: row t, 32 channels
  auto load_z = [&](const uint16_t* zc, uint32_t rows) {
    const __amdgpu_buffer_rsrc_t rsz = make_rsrc(zc, rows * (uint32_t)dim * 2u);
    return __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                     rsz, (uint32_t)((16 * nh + r16) * dim + cb + 8 * g) * 2u, 0, 0));
  };
  // wave 3: dt of a chunk, lane = step
  auto load_dt = [&](const uint16_t* dtc, uint32_t rows) -> uint32_t {
    const __amdgpu_buffer_rsrc_t rsd = make_rsrc(dtc, rows * (uint32_t)H * 2u);
    return lane < kQ ? __builtin_amdgcn_raw_buffer_load_b16(rsd, (uint32_t)(lane * H + h) * 2u, 0, 0)
                     : 0u;
  };

  // ---- per-step values of a chunk (wave 3, lane = step < 32) ----------------
  const float inv_a = coef_is_dt ? 0.0f : 1.0f / Ah;
  auto steps = [&](uint32_t dtbits, int buf) {
    const float dtv = bf16_bits_to_f32(dtbits);
    const float s = prefix32(dtv * A2);
    const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), kQ - 1));
    if (lane < kQ) {
      const float cf = coef_is_dt ? dtv : zoh_coef(dtv, Ah, inv_a);
      sm.ps[buf][0][lane] = s;
      sm.ps[buf][1][lane] = cf;
      sm.ps[buf][2][lane] = fast_exp2(last - s) * cf;
      sm.ps[buf][3][lane] = fast_exp2(s);
    }
  };

  // ---- prologue -------------------------------------------------------------
  // wave 3 keeps the per-step values two chunks ahead: those of chunk c + 2
  // are computed in chunk c's phase A (while waves 0..2 build P) from dt
  // loaded two chunks earlier, into the fourth buffer: its last readers (in
  // chunk c - 2's phase B) are past the previous barrier
  // C is read in phase A, before the chunk's barrier, so it is copied two
  // chunks ahead (into the buffer whose last reader finished before the
  // previous barrier); B^T and x, read in phase B, one chunk ahead.
  uint32_t da = 0, db = 0;  // dt of chunk c + 2 when chunk c starts (wave 3)
  u32x4_t za = {0u, 0u, 0u, 0u};  // z of the chunk
  copy_c(0, cpp);
  copy_c(1, nck_i > 1 ? cpp + kCk : cpp);
  copy_bt(0, btp);
  copy_x(0, xp, rows_of(0));
  if (w == 3) {
    const uint32_t d0 = load_dt(dtp, rows_of(0));
    const uint32_t d1 = load_dt(dtp + dtstep, rows_of(1));
    da = load_dt(dtp + 2 * dtstep, rows_of(2));
    db = load_dt(dtp + 3 * dtstep, rows_of(3));
    steps(d0, 0);
    steps(d1, 1);
  }
  // M tiles two chunks ahead: those of chunk c + 2 are loaded in chunk c's
  // phase B into the registers chunk c's phase A has just read
  f32x4_t mta = zero4, mtb = zero4;
  if constexpr (!PRE) {
    if constexpr (HAS_Z) za = load_z(zp, rows_of(0));
    mta = load_m(mtp);
    mtb = load_m(nck_i > 1 ? mtp + kMk : mtp);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's copies have landed
  __syncthreads();

  // One chunk; the loop runs two per iteration with the registers of z, dt
  // and the M tile swapping roles, so that no register copy waits for a load
  // in flight.
  auto chunk_step = [&](int cc, const u32x4_t& zop, u32x4_t& znext, uint32_t& dtr,
                        f32x4_t& mreg) {
    const int pb = cc & 3;  // per-step values
    const int mb = cc & 1;  // double buffers
    const bool more = cc + 1 < nck_i;

    // ===== phase A ============================================================
    if (w == 3 && cc + 2 < nck_i) steps(dtr, (cc + 2) & 3);
    [[maybe_unused]] f32x4_t ysown = zero4;  // C h_in over this half, row tile nh
    if constexpr (!PRE) {
      // masked weights: tile w of (0,0), (1,0), (1,1)
      if (w < kTiles) {
        const int I = w > 0 ? 1 : 0, J = w == 1 ? 0 : I;
        const float si = sm.ps[pb][0][16 * I + r16];
        const f32x4_t sj = *reinterpret_cast<const f32x4_t*>(&sm.ps[pb][0][16 * J + 4 * g]);
        const f32x4_t cj = *reinterpret_cast<const f32x4_t*>(&sm.ps[pb][1][16 * J + 4 * g]);
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = (I > J || 4 * g + q <= r16) ? mreg[q] * fast_exp2(si - sj[q]) * cj[q] : 0.0f;
        uint32_t h01, l01, h23, l23;
        split_bf16(v[0], v[1], h01, l01);
        split_bf16(v[2], v[3], h23, l23);
        sm.pmh[mb][w][lane] = u32x2_t{h01, h23};
        sm.pml[mb][w][lane] = u32x2_t{l01, l23};
      }
      // C h_in over this wave's state half, both row tiles; the entering
      // state as B operands (slots 0..3 = tile 2k, 4..7 = tile 2k + 1)
      f32x4_t yst[2] = {zero4, zero4};
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        uint32_t hw[4], lw[4];
        split_bf16(st[2 * k][0], st[2 * k][1], hw[0], lw[0]);
        split_bf16(st[2 * k][2], st[2 * k][3], hw[1], lw[1]);
        split_bf16(st[2 * k + 1][0], st[2 * k + 1][1], hw[2], lw[2]);
        split_bf16(st[2 * k + 1][2], st[2 * k + 1][3], hw[3], lw[3]);
        const u32x4_t sh = {hw[0], hw[1], hw[2], hw[3]}, sl = {lw[0], lw[1], lw[2], lw[3]};
        const int pc = nh * (N / 16) + 4 * k + g;  // piece of the C rows
#pragma unroll
        for (int I = 0; I < 2; ++I) {
          const int t = 16 * I + r16;
          const u32x4_t co = lds128(&sm.cs[mb][t * N + 8 * (pc ^ (t & (N / 8 - 1)))]);
          yst[I] = mfma_k32(co, sh, yst[I]);
          yst[I] = mfma_k32(co, sl, yst[I]);
        }
      }
      sm.part[mb][pt][1 - nh][lane] = nh ? yst[0] : yst[1];
      ysown = nh ? yst[1] : yst[0];
    }
    // Every wave's copies of this chunk's operands (issued a chunk ago) have
    // landed before the barrier.  The wait is for all of this wave's vector
    // memory operations: copies into LDS are not ordered with the register
    // loads issued after them, and nothing issued since the last phase B
    // start is still needed later than here.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    // ===== phase B ============================================================
    // dt of chunk c + 3 first, so that waiting for it later does not wait
    // for the copies and stores issued after it
    // dt of chunk c + 4 (wave 3), then the copies: B^T and x of the next
    // chunk, C of the chunk after it (the last chunks' "next" copies read
    // zeros or repeat a chunk into an idle buffer)
    if (w == 3) dtr = load_dt(dtp + 4 * dtstep, rows_of(cc + 4));  // chunk cc + 4
    copy_bt(mb ^ 1, more ? btp + kCk : btp);
    copy_x(mb ^ 1, xp + xstep, rows_of(cc + 1));
    copy_c(mb, cc + 2 < nck_i ? cpp + 2 * kCk : cpp);  // chunk cc + 2
    if constexpr (!PRE) {
      mreg = load_m(cc + 2 < nck_i ? mtp + 2 * kMk : mtp);  // M of chunk cc + 2
      if constexpr (HAS_Z) znext = load_z(zp + xstep, rows_of(cc + 1));
    }
    // x of the chunk in the result layout (exact): xc[tt][q] = x[16 tt + 4g +
    // q][p], q = 0..3, and as packed bf16 (the B operand of P x)
    f32x4_t xc[2];
    u32x2_t xo[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = 16 * tt + r16;
      xc[tt] = mfma_k32(lds128(&sm.xs[mb][t * kBC + 8 * (g ^ swz4(t))]), ipick, zero4);
      xo[tt] = to_bf16x4(xc[tt]);
    }
    auto xval = [&](int tt, int q) { return xc[tt][q]; };
    if constexpr (!PRE) {
      const __amdgpu_buffer_rsrc_t rsy = make_rsrc(yp, rows_of(cc) * (uint32_t)dim * 2u);
      // outputs of row tile I = nh: rows 16 I + 4 g + q, column p
      auto finish = [&](auto row) {
        constexpr int I = decltype(row)::value;
        // in-chunk part P x: row tile 0 has the diagonal tile alone (slots
        // 4..7 zero), row tile 1 the tiles (1,0) and (1,1) in one product
        const u32x2_t z2 = {0u, 0u};
        const u32x4_t ph = cat(sm.pmh[mb][I == 0 ? 0 : 1][lane], I == 0 ? z2 : sm.pmh[mb][2][lane]);
        const u32x4_t pl = cat(sm.pml[mb][I == 0 ? 0 : 1][lane], I == 0 ? z2 : sm.pml[mb][2][lane]);
        const u32x4_t bx = cat(xo[0], xo[1]);
        f32x4_t yin = mfma_k32(ph, bx, zero4);
        yin = mfma_k32(pl, bx, yin);
        const f32x4_t ys = ysown + sm.part[mb][pt][I][lane];
        const f32x4_t e = *reinterpret_cast<const f32x4_t*>(&sm.ps[pb][3][16 * I + 4 * g]);
        f32x4_t zv = zero4;
        if constexpr (HAS_Z) zv = mfma_k32(zop, ipick, zero4);
        float out[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          out[q] = __builtin_fmaf(e[q], ys[q], yin[q]) + Dp * xval(I, q);
          if constexpr (HAS_Z) out[q] *= silu(zv[q]);
        }
        // Store: the bf16 outputs taken as an A operand (row p, slots t)
        // times the identity give the tile transposed in the result layout,
        // lane (row t = 16 I + r16, channels 16 pt + 4 g .. + 3): one 8-byte
        // store per lane instead of four 2-byte ones.  Exact.
        const u32x4_t ya = {pack_bf16(out[0], out[1]), pack_bf16(out[2], out[3]), 0u, 0u};
        const f32x4_t yt = mfma_k32(ya, ipick4, zero4);
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) uint32_t, to_bf16x4(yt)), rsy,
            (uint32_t)r16 * (uint32_t)dim * 2u + (uint32_t)(cb + 16 * pt + 4 * g) * 2u,
            16 * I * dim * 2, 0);
      };
      if (nh)
        finish(std::integral_constant<int, 1>{});
      else
        finish(std::integral_constant<int, 0>{});
    }

    // ---- state update: h <- exp(s_last) h + B^T (w x), this half -----------
    // B operand: w_t x_t[p] (column p, slots as B^T's steps), split
    {
      const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(&sm.ps[pb][2][4 * g]);
      const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(&sm.ps[pb][2][16 + 4 * g]);
      uint32_t hw[4], lw[4];
      split_bf16(w0[0] * xval(0, 0), w0[1] * xval(0, 1), hw[0], lw[0]);
      split_bf16(w0[2] * xval(0, 2), w0[3] * xval(0, 3), hw[1], lw[1]);
      split_bf16(w1[0] * xval(1, 0), w1[1] * xval(1, 1), hw[2], lw[2]);
      split_bf16(w1[2] * xval(1, 2), w1[3] * xval(1, 3), hw[3], lw[3]);
      const u32x4_t wh = {hw[0], hw[1], hw[2], hw[3]}, wl = {lw[0], lw[1], lw[2], lw[3]};
      const float slast = sm.ps[pb][0][kQ - 1];
      const float dec = fast_exp2(slast);
      if constexpr (PRE) dlog += slast;
#pragma unroll
      for (int j = 0; j < NT2; ++j) {
        const int n = nh * (N / 2) + 16 * j + r16;
        const u32x4_t bo = lds128(&sm.bts[mb][n * kQ + 8 * (g ^ swz4(n))]);
        f32x4_t sj = st[j] * dec;
        sj = mfma_k32(bo, wh, sj);
        st[j] = mfma_k32(bo, wl, sj);
      }
    }
    // wave 3: per-step values of chunk c + 2
    // advance to the next chunk
    xp += xstep;
    zp += xstep;
    yp += xstep;
    dtp += dtstep;
    cpp += kCk;
    btp += kCk;
    mtp += kMk;
  };
  u32x4_t zb = {0u, 0u, 0u, 0u};
  for (int cc = 0; cc < nck_i; cc += 2) {
    chunk_step(cc, za, zb, da, mta);
    if (cc + 1 < nck_i) chunk_step(cc + 1, zb, za, db, mtb);
  }

  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no copy into LDS outlives the block
  float* dst = nullptr;
  if (PRE)
    dst = a.ws_hloc + (seg_row * dim + d) * N + soff;
  else if (a.h_last && seg == a.nseg - 1)
    dst = a.h_last + ((size_t)b * dim + d) * N + soff;
  if (dst) {
#pragma unroll
    for (int j = 0; j < NT2; ++j) *reinterpret_cast<f32x4_t*>(dst + 16 * j) = st[j];
  }
  if (PRE && half == 0 && tid == 0) a.ws_dlog[seg_row * H + h] = dlog;
}

// Entering state of each segment: h_in[s + 1] = exp2(dlog[s]) h_in[s] + hloc[s]
// from h_in[0] = h0 (or 0), one thread per (batch row, channel, state);
// consecutive threads take consecutive (channel, state), so every step's
// loads and stores are coalesced rows.
__global__ __launch_bounds__(256) void ssd_carry_kernel(SsdArgs a, int N) {
  const int64_t per_b = (int64_t)a.dim * N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.batch * per_b) return;
  const int64_t b = i / per_b, dn = i % per_b;
  const int h = (int)(dn / N) / kHD;
  float v = a.h0 ? a.h0[i] : 0.0f;
  for (int s = 0; s + 1 < a.nseg; ++s) {
    const size_t row = (size_t)b * a.nseg + s;
    v = __builtin_fmaf(fast_exp2(a.ws_dlog[row * a.nheads + h]), v, a.ws_hloc[row * per_b + dn]);
    a.ws_hin[(row + 1) * per_b + dn] = v;
  }
}

constexpr int64_t kMaxRows = 65535;  // grid.y limit

template <int N>
hipError_t launch_prep(SsdArgs a, hipStream_t stream) {
  for (int64_t r0 = 0; r0 < a.batch; r0 += kMaxRows) {
    a.row0 = r0;
    const int rows = (int)(a.batch - r0 < kMaxRows ? a.batch - r0 : kMaxRows);
    hipLaunchKernelGGL(ssd_prep_kernel<N>, dim3((unsigned)a.nck, rows), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int N, bool HAS_Z, bool EULER, bool PRE>
hipError_t launch_ssd_pass(SsdArgs a, int segs, hipStream_t stream) {
  auto kern = ssd_scan_kernel<N, HAS_Z, EULER, PRE>;
  const size_t smem = sizeof(SsdSmem<N>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  for (int64_t r0 = 0; r0 < a.batch; r0 += kMaxRows) {
    a.row0 = r0;
    const int rows = (int)(a.batch - r0 < kMaxRows ? a.batch - r0 : kMaxRows);
    hipLaunchKernelGGL(kern, dim3(2 * a.nheads, rows, segs), dim3(kSsdThreads), smem, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int N, bool HAS_Z, bool EULER>
hipError_t launch_ssd_t(const SsdArgs& a, hipStream_t stream) {
  hipError_t e = launch_prep<N>(a, stream);
  if (e != hipSuccess) return e;
  if (a.nseg > 1) {
    e = launch_ssd_pass<N, HAS_Z, EULER, true>(a, a.nseg - 1, stream);
    if (e != hipSuccess) return e;
    const int64_t n = a.batch * (int64_t)a.dim * N;
    hipLaunchKernelGGL(ssd_carry_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       a, N);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_ssd_pass<N, HAS_Z, EULER, false>(a, a.nseg, stream);
}

template <int N>
hipError_t launch_ssd_n(const SsdArgs& a, hipStream_t stream) {
  if (a.z) return a.euler ? launch_ssd_t<N, true, true>(a, stream)
                          : launch_ssd_t<N, true, false>(a, stream);
  return a.euler ? launch_ssd_t<N, false, true>(a, stream)
                 : launch_ssd_t<N, false, false>(a, stream);
}

}  // namespace

bool ssd_supported(int64_t headdim, int64_t dstate) {
  return headdim == kHD && (dstate == 64 || dstate == 128);
}

SsdLayout ssd_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t nheads, int64_t dstate,
                     int nseg) {
  auto align = [](size_t v) { return (v + 255) & ~size_t(255); };
  SsdLayout l{};
  const size_t nck = (size_t)((seqlen + kQ - 1) / kQ);
  const size_t rows = (size_t)batch * nck * kQ * dstate * sizeof(uint16_t);  // C or B^T
  l.cp_off = 0;
  l.bt_off = align(rows);
  l.mt_off = l.bt_off + align(rows);
  l.total = l.mt_off + align((size_t)batch * nck * kTiles * kWave * 4 * sizeof(float));
  if (nseg > 1) {
    const size_t st = align((size_t)batch * nseg * dim * dstate * sizeof(float));
    l.hloc_off = l.total;
    l.hin_off = l.hloc_off + st;
    l.dlog_off = l.hin_off + st;
    l.total = l.dlog_off + align((size_t)batch * nseg * nheads * sizeof(float));
  }
  return l;
}

hipError_t launch_ssd(const SsdArgs& a, int dstate, hipStream_t stream) {
  switch (dstate) {
    case 64: return launch_ssd_n<64>(a, stream);
    case 128: return launch_ssd_n<128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssm
