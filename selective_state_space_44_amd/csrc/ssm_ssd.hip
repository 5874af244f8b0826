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
//   y_i   = sum_{j<=i} (C_i . B_j) exp(s_i - s_j) coef_j x_j      in-chunk part
//         + exp(s_i) C_i . h_in                                   entering state
//   h_out = exp(s_last) h_in + sum_j exp(s_last - s_j) coef_j x_j B_j^T
//
// and y = (y + D x) * SiLU(z).  Each sum is a matrix product:
//   * M = C B^T per chunk (32 x 32, contraction over the N states),
//   * Y_in = P X with P = M masked to j <= i and weighted by
//     exp(s_i - s_j) coef_j (contraction over the chunk's steps),
//   * Y_state = C h_in^T (contraction over the states),
//   * h_out^T = B^T (w x) with w_t = exp(s_last - s_t) coef_t (contraction
//     over the steps).
//
// Organisation: one block per (half head of 32 channels, batch row) walks
// 32-step chunks in order, so the state never leaves the registers and no
// carry pass exists.  Its 4 waves are 2 channel tiles x 2 state halves: wave
// (pt, nh) holds the state h[n][p] of channels p = 16pt..16pt+15 and states
// n in half nh as N/32 MFMA accumulator tiles, updates them, and computes
// C h over its half for the chunk's two 16-step row tiles; it finishes row
// tile nh (its partial plus the other half's, passed through LDS).  The
// chunk's 32 x 32 matrix P has three lower-triangular 16 x 16 tiles, one on
// each of waves 0..2, passed through LDS.  At the Mamba-2-like shape (4 x 80
// heads) this makes 640 blocks of 32.5 KB LDS (N = 128), all resident at once
// (2-3 per CU).
//
// Data movement per chunk: the chunk's x, z (32 steps x 32 channels), B, C
// (32 steps x N) and dt are loaded into registers two chunks ahead and
// staged in LDS in their natural layout.  The operand layouts the
// contractions need -- x and B with the step index contiguous, x and z in the
// result layout of the epilogue -- come from products with an identity
// matrix (see identity_pick), and the outputs are transposed the same way
// for 8-byte stores.  The decay exponents of a chunk (a prefix sum over its
// steps) are computed one chunk ahead by the wave that has no P tile.  Three
// barriers per chunk: staging written; P and the partial C h written; (next
// chunk) all reads done.
//
// Precision: B, C and x are bf16 inputs, exact as MFMA operands.  The other
// operands -- the masked weights P, the state h and the weighted inputs w x --
// are fp32 values; each is split into a bf16 high part and a bf16 low part
// (v = hi + lo to about 2^-17 |v|) and both parts are multiplied, so every
// product carries ~16 significant bits and all sums are fp32.  The state
// stays fp32 between chunks.
//
// MFMA lane layouts used (v_mfma_f32_16x16x32_bf16 only; 16 x 16 tiles, lane
// l, g = l / 16):
//   A operand: row l % 16, k slots 8g..8g+7
//   B operand: column l % 16, the same k slots
//   result:    column l % 16, rows 4g..4g+3
// Only the row / column / result layout matters: a product pairs the k
// slots of A and B one to one, so any permutation of the contraction index
// applied to both operands gives the same sum.  The kernel uses that freedom
// where a result tile becomes the next product's operand without a trip
// through LDS (the state as the B operand of C h^T, the identity products).
// The 16x16x16 form is not used: in one compiled schedule the result rows
// 0-1 of such a product were read before it had completed.

#include "ssm_device.h"
#include "ssm_launch.h"
#include "ssm_mfma.h"

namespace ssm {
namespace {

constexpr int kQ = 32;            // steps per chunk
constexpr int kHD = 64;           // channels per head
constexpr int kBC = 32;           // channels per block (half a head)
constexpr int kSsdThreads = 256;  // 4 waves: 2 channel tiles x 2 state halves
constexpr int kRowT = kQ + 8;     // bf16 per row of P: 80 B, so 8 consecutive
                                  // rows start on distinct banks
constexpr int kRowX = kBC + 8;    // bf16 per row of the staged x and z

template <int N>
struct SsdSmem {
  static constexpr int kRowN = N + 8;    // bf16 per state-contiguous row
  alignas(16) uint16_t cs[kQ][kRowN];    // C of the chunk, [t][n]
  alignas(16) uint16_t bs[kQ][kRowN];    // B, [t][n]
  alignas(16) uint16_t xs[kQ][kRowX];    // x of the block's channels, [t][p]
  alignas(16) uint16_t zs[kQ][kRowX];    // z, [t][p]
  alignas(16) uint16_t pmh[kQ][kRowT];   // masked weights P[i][j], high part
  alignas(16) uint16_t pml[kQ][kRowT];   // low part
  // C h over one state half, for the row tile the other half's wave finishes:
  // [channel tile][row tile][lane][result register]
  alignas(16) float part[2][2][kWave][4];
  // per-step values of the chunk (two buffers: the next chunk's are
  // computed while the current one runs)
  alignas(16) float s2[2][kQ];     // s_t * log2(e)
  alignas(16) float coef[2][kQ];   // coef_t
  alignas(16) float wgt[2][kQ];    // exp(s_last - s_t) coef_t
  alignas(16) float ein[2][kQ];    // exp(s_t)
};

// PRE: the state-only pass over segments 0..nseg-2 (no outputs): end state
// from zero and the log2 of the segment's decay, into the workspace.
template <int N, bool HAS_Z, bool EULER, bool PRE>
__global__ __launch_bounds__(kSsdThreads) __attribute__((amdgpu_waves_per_eu(3)))
void ssd_scan_kernel(SsdArgs a) {
  constexpr int NT2 = N / 32;   // state tiles per wave (half of the N/16)
  constexpr int NK = N / 64;    // 32-state contraction steps per state half
  constexpr int NB = N / 8;     // B / C columns staged by each thread
  constexpr int NBV = NB / 8;   // 16-byte pieces of them
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
  const int pt = w & 1, nh = w >> 1;           // channel tile, state half (= row tile)
  const int dim = a.dim;
  const int64_t L = a.seqlen;
  const float Ah = a.A[h];
  const float A2 = Ah * kLog2e;
  const bool coef_is_dt = EULER || Ah == 0.0f;  // the Euler rule, or the hold's a -> 0 limit
  const int cb = h * kHD + kBC * half;          // first channel of the block
  const int p = 16 * pt + r16;                  // this lane's channel in the block
  const int d = cb + p;
  const float Dp = a.Dskip ? a.Dskip[d] : 0.0f;
  const int ts = tid & (kQ - 1), cg = tid >> 5;  // staging: step, column group
  // this block's steps [tb, te)
  const int seg = blockIdx.z;
  const int64_t tb = (int64_t)seg * a.seg_len;
  const int64_t te = tb + a.seg_len < L ? tb + a.seg_len : L;
  const size_t seg_row = (size_t)b * a.nseg + seg;  // (batch row, segment) of the workspace
  const size_t soff = 16 * nh * NT2 + 4 * g;        // this lane's first state

  // state tile j: st[j][q] = h[n = 16 (nh NT2 + j) + 4 g + q][p]
  f32x4_t st[NT2];
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
  float dlog = 0.0f;  // PRE: log2 of the segment's decay

  const u32x4_t ipick[2] = {identity_pick(0, r16, g), identity_pick(16, r16, g)};
  const u32x4_t ipick4 = identity_pick4(r16, g);

  // Staging registers: thread (ts, cg) holds step ts of a chunk -- channels
  // 4cg..4cg+3 of the block for x and z, states NB cg .. NB cg + NB - 1 of B
  // and C, and (wave 3, lanes < kQ) dt.  Two sets: the loads of chunk c + 2
  // are issued while chunk c runs.  Rows past the end of the sequence read as
  // zero (buffer bounds): steps with dt = 0, which leave the state unchanged,
  // and whose outputs are not stored.
  struct Stage {
    u32x2_t x, z;
    u32x4_t b[NBV], c[NBV];
    uint32_t dt;
  };
  auto fetch = [&](Stage& sg, int64_t t0) {
    const uint32_t rows = (uint32_t)(te - t0 < kQ ? te - t0 : (int64_t)kQ);
    if (w == 3) {
      const __amdgpu_buffer_rsrc_t rsd = make_rsrc(
          static_cast<const uint16_t*>(a.dt) + (b * L + t0) * H, rows * (uint32_t)H * 2u);
      sg.dt = lane < kQ
                  ? __builtin_amdgcn_raw_buffer_load_b16(rsd, (uint32_t)lane * H * 2u + h * 2u, 0, 0)
                  : 0u;
    }
    const uint32_t ox = (uint32_t)ts * (uint32_t)dim * 2u + (uint32_t)(cb + 4 * cg) * 2u;
    const __amdgpu_buffer_rsrc_t rsx = make_rsrc(
        static_cast<const uint16_t*>(a.x) + (b * L + t0) * dim, rows * (uint32_t)dim * 2u);
    sg.x = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rsx, ox, 0, 0));
    if constexpr (HAS_Z && !PRE) {
      const __amdgpu_buffer_rsrc_t rsz = make_rsrc(
          static_cast<const uint16_t*>(a.z) + (b * L + t0) * dim, rows * (uint32_t)dim * 2u);
      sg.z = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rsz, ox, 0, 0));
    }
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(static_cast<const uint16_t*>(a.B) + (b * L + t0) * N, rows * N * 2u);
    const __amdgpu_buffer_rsrc_t rsc =
        make_rsrc(static_cast<const uint16_t*>(a.C) + (b * L + t0) * N, rows * N * 2u);
    const uint32_t ob = (uint32_t)ts * N * 2u + (uint32_t)(NB * cg) * 2u;
#pragma unroll
    for (int j = 0; j < NBV; ++j) {
      sg.b[j] = __builtin_bit_cast(u32x4_t,
                                   __builtin_amdgcn_raw_buffer_load_b128(rsb, ob + 16u * j, 0, 0));
      if constexpr (!PRE)
        sg.c[j] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsc, ob + 16u * j, 0, 0));
    }
  };
  // wave 3: the chunk's decay exponents (inclusive prefix sum of a * dt over
  // its steps, lanes < kQ) and per-step weights, into buffer `buf`
  auto scan = [&](const Stage& sg, int buf) {
    const float dtv = bf16_bits_to_f32(sg.dt);
    float s = dtv * A2;
#pragma unroll
    for (int o = 1; o < kQ; o <<= 1) {
      const float v = __shfl_up(s, o);
      if (lane >= o) s += v;
    }
    const float last = __shfl(s, kQ - 1);
    if (lane < kQ) {
      const float cf = coef_is_dt ? dtv : expm1f(dtv * Ah) / Ah;
      sm.s2[buf][lane] = s;
      sm.coef[buf][lane] = cf;
      sm.wgt[buf][lane] = fast_exp2(last - s) * cf;
      sm.ein[buf][lane] = fast_exp2(s);
    }
  };

  const int64_t nck = (te - tb + kQ - 1) / kQ;
  auto chunk = [&](int64_t c, Stage& cur, const Stage& nxt) {
    const int64_t t0 = tb + c * kQ;
    const int buf = (int)(c & 1);
    __syncthreads();  // every read of the previous chunk's LDS is done

    // ---- stage the chunk in natural layout ----------------------------
    *reinterpret_cast<u32x2_t*>(&sm.xs[ts][4 * cg]) = cur.x;
    if constexpr (HAS_Z && !PRE) *reinterpret_cast<u32x2_t*>(&sm.zs[ts][4 * cg]) = cur.z;
#pragma unroll
    for (int j = 0; j < NBV; ++j) {
      *reinterpret_cast<u32x4_t*>(&sm.bs[ts][NB * cg + 8 * j]) = cur.b[j];
      if constexpr (!PRE) *reinterpret_cast<u32x4_t*>(&sm.cs[ts][NB * cg + 8 * j]) = cur.c[j];
    }
    __syncthreads();

    if (c + 2 < nck) fetch(cur, t0 + 2 * kQ);

    if (!PRE && w < 3) {
      // ---- masked weights P: tiles (0,0), (1,0), (1,1) on waves 0..2 ----
      const int I = w > 0 ? 1 : 0, J = w == 1 ? 0 : I;
      // M^T tile: rows j (B rows), columns i (C rows), contraction over states
      f32x4_t m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < N / 32; ++k)
        m = mfma_k32(lds128(&sm.bs[16 * J + r16][32 * k + 8 * g]),
                     lds128(&sm.cs[16 * I + r16][32 * k + 8 * g]), m);
      // m[q] = C_i . B_j with i = 16 I + r16, j = 16 J + 4 g + q
      const int i = 16 * I + r16;
      const float si = sm.s2[buf][i];
      const f32x4_t sj = *reinterpret_cast<const f32x4_t*>(&sm.s2[buf][16 * J + 4 * g]);
      const f32x4_t cj = *reinterpret_cast<const f32x4_t*>(&sm.coef[buf][16 * J + 4 * g]);
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = 16 * J + 4 * g + q;
        v[q] = (j <= i) ? m[q] * fast_exp2(si - sj[q]) * cj[q] : 0.0f;
      }
      uint32_t h0w, l0w, h1w, l1w;
      split_bf16(v[0], v[1], h0w, l0w);
      split_bf16(v[2], v[3], h1w, l1w);
      *reinterpret_cast<u32x2_t*>(&sm.pmh[i][16 * J + 4 * g]) = u32x2_t{h0w, h1w};
      *reinterpret_cast<u32x2_t*>(&sm.pml[i][16 * J + 4 * g]) = u32x2_t{l0w, l1w};
    } else if (w == 3 && c + 1 < nck) {
      scan(nxt, buf ^ 1);  // wave 3: the next chunk's per-step values
    }

    f32x4_t yst[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if constexpr (!PRE) {
    // ---- C h over this wave's state half, both row tiles ----------------
    // the entering state as B operands: slots 0..3 = tile 2k, 4..7 = tile
    // 2k + 1 of the half (states nh N/2 + 32k + 4g + q and + 16)
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      uint32_t hw[4], lw[4];
      split_bf16(st[2 * k][0], st[2 * k][1], hw[0], lw[0]);
      split_bf16(st[2 * k][2], st[2 * k][3], hw[1], lw[1]);
      split_bf16(st[2 * k + 1][0], st[2 * k + 1][1], hw[2], lw[2]);
      split_bf16(st[2 * k + 1][2], st[2 * k + 1][3], hw[3], lw[3]);
      const u32x4_t sh = {hw[0], hw[1], hw[2], hw[3]}, sl = {lw[0], lw[1], lw[2], lw[3]};
      const int n0 = nh * (N / 2) + 32 * k + 4 * g;
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const u32x4_t co = cat(lds64(&sm.cs[16 * I + r16][n0]), lds64(&sm.cs[16 * I + r16][n0 + 16]));
        yst[I] = mfma_k32(co, sh, yst[I]);
        yst[I] = mfma_k32(co, sl, yst[I]);
      }
    }
    // the other half's wave finishes row tile 1 - nh
    *reinterpret_cast<f32x4_t*>(&sm.part[pt][1 - nh][lane][0]) = nh ? yst[0] : yst[1];
    __syncthreads();
    }

    // ---- x (and z) of this wave's channels in result layout ------------
    // xc[tt][q] = x[16 tt + 4 g + q][p], exact, from identity products
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4_t xc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) xc[tt] = mfma_k32(lds128(&sm.xs[16 * tt + r16][8 * g]), ipick[pt], zero4);

    if constexpr (!PRE) {
    // ---- outputs of row tile I = nh for this wave's 16 channels ---------
    {
      const int I = nh, i = 16 * I + r16;
      // in-chunk part P x: row tile 0 has the diagonal tile alone (slots
      // 4..7 zero), row tile 1 the tiles 0 and 1 in one product; x as the B
      // operand (column p, slots j = 4g + q and 16 + 4g + q)
      const u32x2_t zero = {0u, 0u};
      const u32x4_t xo = cat(to_bf16x4(xc[0]), I ? to_bf16x4(xc[1]) : zero);
      f32x4_t yin = mfma_k32(cat(lds64(&sm.pmh[i][4 * g]), I ? lds64(&sm.pmh[i][16 + 4 * g]) : zero),
                             xo, zero4);
      yin = mfma_k32(cat(lds64(&sm.pml[i][4 * g]), I ? lds64(&sm.pml[i][16 + 4 * g]) : zero), xo,
                     yin);
      const f32x4_t other = *reinterpret_cast<const f32x4_t*>(&sm.part[pt][I][lane][0]);
      const f32x4_t ys = (nh ? yst[1] : yst[0]) + other;
      // epilogue: rows 16 I + 4 g + q, column p
      const f32x4_t e = *reinterpret_cast<const f32x4_t*>(&sm.ein[buf][16 * I + 4 * g]);
      const f32x4_t xv = nh ? xc[1] : xc[0];
      f32x4_t zv = zero4;
      if constexpr (HAS_Z) zv = mfma_k32(lds128(&sm.zs[16 * I + r16][8 * g]), ipick[pt], zero4);
      float out[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        out[q] = __builtin_fmaf(e[q], ys[q], yin[q]) + Dp * xv[q];
        if constexpr (HAS_Z) out[q] *= silu(zv[q]);
      }
      // Store: the bf16 outputs (rows 16 I + 4 g + q, column p) taken as an
      // A operand (row p, slots t) times the identity give the tile
      // transposed in the result layout, lane (row t = 16 I + r16, channels
      // 16 pt + 4 g .. + 3): one 8-byte store per lane instead of four
      // 2-byte ones.  Exact (bf16 values times 1).
      const u32x4_t ya = {pack_bf16(out[0], out[1]), pack_bf16(out[2], out[3]), 0u, 0u};
      const f32x4_t yt = mfma_k32(ya, ipick4, zero4);
      const uint32_t rows = (uint32_t)(L - t0 < kQ ? L - t0 : (int64_t)kQ);
      const __amdgpu_buffer_rsrc_t rsy =
          make_rsrc(static_cast<uint16_t*>(a.y) + (b * L + t0) * dim, rows * (uint32_t)dim * 2u);
      __builtin_amdgcn_raw_buffer_store_b64(
          __builtin_bit_cast(__attribute__((ext_vector_type(2))) uint32_t, to_bf16x4(yt)), rsy,
          (uint32_t)(16 * I + r16) * (uint32_t)dim * 2u + (uint32_t)(cb + 16 * pt + 4 * g) * 2u, 0,
          0);
    }
    }

    // ---- state update: h <- exp(s_last) h + (w x)^T B, this half --------
    // B operand: w_t x_t[p] (column p, slots t = 4g + q and 16 + 4g + q),
    // split into bf16 high and low parts
    u32x4_t wh, wl;
    {
      const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(&sm.wgt[buf][4 * g]);
      const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(&sm.wgt[buf][16 + 4 * g]);
      uint32_t hw[4], lw[4];
      split_bf16(w0[0] * xc[0][0], w0[1] * xc[0][1], hw[0], lw[0]);
      split_bf16(w0[2] * xc[0][2], w0[3] * xc[0][3], hw[1], lw[1]);
      split_bf16(w1[0] * xc[1][0], w1[1] * xc[1][1], hw[2], lw[2]);
      split_bf16(w1[2] * xc[1][2], w1[3] * xc[1][3], hw[3], lw[3]);
      wh = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
      wl = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
    }
    const float dec = fast_exp2(sm.s2[buf][kQ - 1]);
    if constexpr (PRE) dlog += sm.s2[buf][kQ - 1];
#pragma unroll
    for (int j2 = 0; j2 < NT2 / 2; ++j2) {
      // states 32 n32 .. 32 n32 + 31 (two tiles of this half) of B, rows t
      const int n32 = nh * (NT2 / 2) + j2;
      const u32x4_t b0 = lds128(&sm.bs[r16][32 * n32 + 8 * g]);
      const u32x4_t b1 = lds128(&sm.bs[16 + r16][32 * n32 + 8 * g]);
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        // A operand: row n = 32 n32 + 16 o + r16, slots t (B transposed by
        // identity products, exact)
        const u32x4_t bo = cat(to_bf16x4(mfma_k32(b0, ipick[o], zero4)),
                               to_bf16x4(mfma_k32(b1, ipick[o], zero4)));
        f32x4_t& sj = st[2 * j2 + o];
        sj *= dec;
        sj = mfma_k32(bo, wh, sj);
        sj = mfma_k32(bo, wl, sj);
      }
    }
  };

  Stage sa, sb;
  sb.dt = 0u;
  fetch(sa, tb);
  if (nck > 1) fetch(sb, tb + kQ);
  if (w == 3) scan(sa, 0);
  for (int64_t c = 0; c < nck; c += 2) {
    chunk(c, sa, sb);
    if (c + 1 < nck) chunk(c + 1, sb, sa);
  }

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

template <int N, bool HAS_Z, bool EULER, bool PRE>
hipError_t launch_ssd_pass(SsdArgs a, int segs, hipStream_t stream) {
  auto kern = ssd_scan_kernel<N, HAS_Z, EULER, PRE>;
  const size_t smem = sizeof(SsdSmem<N>);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  constexpr int64_t kMaxRows = 65535;  // grid.y limit
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
  if (a.nseg > 1) {
    hipError_t e = launch_ssd_pass<N, HAS_Z, EULER, true>(a, a.nseg - 1, stream);
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

size_t ssd_workspace_bytes(int64_t batch, int64_t dim, int64_t nheads, int64_t dstate,
                           int nseg) {
  if (nseg <= 1) return 0;
  auto align = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t st = (size_t)batch * nseg * dim * dstate * sizeof(float);
  return 2 * align(st) + align((size_t)batch * nseg * nheads * sizeof(float));
}

size_t ssd_smem_bytes(int64_t dstate) {
  return dstate == 64 ? sizeof(SsdSmem<64>) : sizeof(SsdSmem<128>);
}

hipError_t launch_ssd(const SsdArgs& a, int dstate, hipStream_t stream) {
  switch (dstate) {
    case 64: return launch_ssd_n<64>(a, stream);
    case 128: return launch_ssd_n<128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssm
