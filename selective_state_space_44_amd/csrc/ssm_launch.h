// ssm_launch.h -- internal interface between the C ABI (ssm_abi.cpp) and the
// HIP kernels (ssm_scan.hip, ssm_decode.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

// Prologue of the fused scan: x = act(causal depthwise conv1d(x_raw) + conv_b)
// and delta = softplus(delta_raw + delta_bias).  d_conv == 0: no prologue
// (x and delta are used as given).
struct Prologue {
  const float* conv_w;      // [dim, d_conv], tap d_conv-1 multiplies the current step
  const float* conv_b;      // [dim], nullable
  const float* delta_bias;  // [dim], nullable
  int d_conv;               // 0 (no prologue) or 1..4
  int conv_silu;            // SiLU after the convolution
};

// Everything a scan launch needs.  Sizes are validated by the ABI layer.
struct ScanArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;  // nullable
  const void* z;       // nullable
  const float* h0;     // nullable
  void* y;
  float* h_last;       // nullable
  // carry workspace (only when nchunks > 1)
  float* ws_hloc;      // [batch, nchunks, dim, 16]  chunk-local end state from zero
  float* ws_hin;       // [batch, nchunks, dim, 16]  state entering each chunk
  double* ws_sdelta;   // [batch, nchunks, dim]      sum of delta over each chunk
  int64_t seqlen;
  int64_t chunk_len;
  int dim;
  int batch;
  int nchunks;
  Prologue pro;        // x and delta above are x_raw and delta_raw when pro.d_conv > 0
  int a_per_channel;   // A is [dim] (one value per channel) instead of [dim, 16]
  int euler;           // Bbar = delta * B instead of the zero-order hold
};

struct DecodeArgs {
  float* h;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;  // nullable
  const void* z;       // nullable
  void* y;
  int64_t batch;
  int dim;
  int64_t row0;        // first batch row of this launch (set by launch_decode)
  int dstate;          // 16, 32, 64 or 128
  int a_per_channel;   // A is [dim] (one value per channel)
  int euler;           // Bbar = delta * B instead of the zero-order hold
};

// Steps per tile of the scan kernels; chunks start on a tile boundary.
int scan_tile_steps();

// Byte layout of the scan workspace: the per-chunk carry state (empty when
// nchunks <= 1).
struct ScanWorkspace {
  size_t hloc_off, hin_off, sdelta_off, total;
};
ScanWorkspace scan_workspace_layout(int64_t batch, int64_t dim, int nchunks);

// Enqueue a scan.  io_bf16 selects the I/O type; waves_per_group is one of
// 2, 4, 8, 16.  With nchunks > 1 the default schedule takes two launches:
//   phase bit 1 -- the first launch (main pass of chunk 0, writing its y and
//                  the state entering chunk 1, beside carry pass 1 of chunks
//                  1 .. K-2) and carry pass 2;
//   phase bit 2 -- the main pass of chunks 1 .. K-1.
// With kPhaseThreePass also set, the three-pass schedule runs instead:
//   bit 1 -- carry pass 1 on chunks 0 .. K-2 and carry pass 2 from h0 (the
//            state entering every chunk, nothing else written: the backward
//            uses this);
//   bit 2 -- the main pass of every chunk.
// Returns hipSuccess or the launch error.
constexpr int kPhaseThreePass = 4;
hipError_t launch_scan(const ScanArgs& a, bool io_bf16, int waves_per_group, int phase,
                       hipStream_t stream);

// Enqueue the cross-chunk composition alone: ws_in[c] = state entering chunk
// c, from init (nullable = 0) and each chunk's local result ws_loc and delta
// sum ws_sdelta (layouts as ScanArgs).  reverse: from the last chunk to the
// first.
hipError_t launch_carry(const float* A, int a_per_channel, const float* init,
                        const float* ws_loc, const double* ws_sdelta, float* ws_in, int batch,
                        int dim, int nchunks, bool reverse, hipStream_t stream);

// Backward of the scan.  Forward inputs as ScanArgs (x, delta, A, B, C,
// Dskip, z, h0, variant flags; chunk_len <= kBwdChunk, nchunks chunks);
// dy, dh_last (nullable) the upstream gradients; outputs dx, ddelta, dz
// (IO type, dz only with z), dA (fp32, [dim, 16] or [dim]), dB, dC (IO type),
// dD, dh0 (fp32, nullable).
constexpr int kBwdChunk = 32;
struct BwdArgs {
  ScanArgs f;
  const void* dy;
  const float* dh_last;
  void* dx;
  void* ddelta;
  void* dz;
  float* dA;
  void* dB;
  void* dC;
  float* dD;
  float* dh0;
  // workspace pieces
  float* ws_eloc;     // [batch, nchunks, dim, 16]  chunk-local adjoint from zero
  float* ws_ein;      // [batch, nchunks, dim, 16]  adjoint entering each chunk from the right
  double* ws_sdr;     // [batch, nchunks, dim]      delta sum of each chunk
  float* ws_pdB;      // [batch, groups, seqlen, 16] per 64-channel group
  float* ws_pdC;      // [batch, groups, seqlen, 16]
  float* ws_pdA;      // [batch, nchunks, dim, 16]
  float* ws_pdD;      // [batch, nchunks, dim]
  // Larger states run as 16-state slices (see launch_scan_bwd_sliced).  When
  // acc_dx is set, the main kernel adds its per-(t, d) results into these
  // fp32 [batch, seqlen, dim] buffers (dx with the D term, ddelta, and C.h of
  // the slice when z is given) instead of storing dx, ddelta and dz.
  float* acc_dx;
  float* acc_dd;
  float* acc_sp;
  // placement of dB, dC ([.., bc_ld] rows, from column bc_col0) and of a
  // per-state dA ([dim, a_ld] rows, from column a_col0); 0 = 16 / 0.  With A
  // per channel, a_accumulate adds the slice's dA to dA instead of storing it.
  int64_t bc_ld;
  int bc_col0;
  int64_t a_ld;
  int a_col0;
  int a_accumulate;
};
struct BwdWorkspace {
  ScanWorkspace fwd, rev;
  size_t rev_base, pdB_off, pdC_off, pdA_off, pdD_off, total;
};
BwdWorkspace bwd_workspace_layout(int64_t batch, int64_t seqlen, int64_t dim, int nchunks);
hipError_t launch_scan_bwd(const BwdArgs& a, bool io_bf16, hipStream_t stream);

// Backward for 32, 64 or 128 states: the states of a channel evolve
// independently and meet only in sums over n (y, and through it dx, ddelta
// and dz), so the 16-state backward runs on each 16-state slice -- B, C, A,
// h0 and dh_last slices gathered into the workspace -- with its per-(t, d)
// results accumulated in fp32, and a last kernel writes dx, ddelta and dz.
struct BwdSliceWorkspace {
  BwdWorkspace base;  // of one 16-state slice
  size_t bs_off, cs_off, as_off, h0s_off, dhls_off, dh0s_off;
  size_t accx_off, accd_off, accs_off, total;
};
BwdSliceWorkspace bwd_slice_layout(int64_t batch, int64_t seqlen, int64_t dim, int nchunks,
                                   int io_bytes);
// `a` holds the full problem (dstate states) with the workspace pointers of
// one slice set up as for the 16-state backward; `wsb` is the workspace base.
hipError_t launch_scan_bwd_sliced(const BwdArgs& a, int dstate, bool io_bf16, char* wsb,
                                  const BwdSliceWorkspace& w, hipStream_t stream);

// Head <-> channel maps of the step and decay shared per head:
// out[r, h * P + p] = in[r, h] (elements of 2 or 4 bytes), and
// out[r, h] = sum over p of in[r, h * P + p] (fp32 in; out_kind 1 = bf16,
// 0 = fp32).
hipError_t launch_repeat_heads(const void* in, void* out, int64_t rows, int heads, int P,
                               int elem_bytes, hipStream_t stream);
hipError_t launch_sum_heads(const float* in, void* out, int64_t rows, int heads, int P,
                            int out_kind, hipStream_t stream);

// Scan for state sizes 32, 64, 128: one pass over the sequence, no
// workspace (chunk fields of ScanArgs unused; no prologue).
bool scan_wide_supported(int64_t dstate);
hipError_t launch_scan_wide(const ScanArgs& a, int dstate, bool io_bf16, hipStream_t stream);

// Scan with the step and decay rate shared by each head of 64 channels, in
// its masked-matrix form on the matrix cores (ssm_ssd.hip).  bf16 x, dt, B,
// C, z, y; fp32 A [nheads], Dskip [dim], h0 / h_last [batch, dim, dstate].
constexpr int kSsdChunk = 32;  // steps per chunk of the masked-matrix scan
struct SsdArgs {
  const void* x;       // [batch, seqlen, dim]
  const void* dt;      // [batch, seqlen, nheads]
  const float* A;      // [nheads]
  const void* B;       // [batch, seqlen, dstate]
  const void* C;
  const float* Dskip;  // nullable
  const void* z;       // nullable
  const float* h0;     // nullable
  void* y;
  float* h_last;       // nullable
  int64_t seqlen;
  int64_t batch;
  int64_t row0;        // first batch row of a launch (set by launch_ssd)
  int nheads;
  int dim;             // nheads * 64
  int euler;
  // Per (batch row, chunk) operands shared by every head, written by a
  // pre-pass: C with its states reordered, B^T and the lower-triangular
  // tiles of C B^T.
  int64_t nck;         // ceil(seqlen / kSsdChunk)
  void* ws_cp;         // [batch, nck, kSsdChunk, dstate] bf16
  void* ws_bt;         // [batch, nck, dstate, kSsdChunk] bf16
  float* ws_mt;        // [batch, nck, 3, 64, 4]
  // Sequence segments run by separate blocks (nseg > 1): a state-only pass
  // writes each segment's end state from zero and the log2 of its decay, a
  // carry composes them in order, and the main pass starts every segment from
  // its entering state.
  int nseg;            // 1 = one block walks the whole sequence
  int64_t seg_len;     // steps per segment, a multiple of kSsdChunk
  float* ws_hloc;      // [batch, nseg, dim, dstate]
  float* ws_hin;       // [batch, nseg, dim, dstate] (segment 0 unused)
  float* ws_dlog;      // [batch, nseg, nheads]
};
// Workspace of the masked-matrix scan (byte offsets; segment buffers only
// when nseg > 1).
struct SsdLayout {
  size_t cp_off, bt_off, mt_off, hloc_off, hin_off, dlog_off, total;
};
SsdLayout ssd_layout(int64_t batch, int64_t seqlen, int64_t dim, int64_t nheads, int64_t dstate,
                     int nseg);

// Backward of the per-head scan in its masked-matrix form, chunk-parallel
// (64-channel heads, 64 or 128 states, bf16 I/O).  Workspace carved by
// ssd_bwd_mm_layout.
struct SsdBwdArgs {
  const void* x;        // [batch, seqlen, dim] bf16
  const void* dt;       // [batch, seqlen, nheads]
  const float* A;       // [nheads]
  const void* B;        // [batch, seqlen, dstate]
  const void* C;
  const float* Dskip;   // nullable
  const void* z;        // nullable
  const float* h0;      // nullable
  const void* dy;       // [batch, seqlen, dim]
  const float* dh_last; // nullable
  void* dx;
  void* ddt;            // [batch, seqlen, nheads]
  float* dA;            // [nheads]
  void* dB;
  void* dC;
  float* dD;            // nullable
  void* dz;             // nullable (with z)
  float* dh0;           // [batch, dim, dstate]: the output, or workspace scratch
  int64_t seqlen;
  int64_t batch;
  int nheads;
  int dim;
  int dstate;
  int euler;
  int nchunks;          // ceil(seqlen / 32)
  int ngroups;          // ceil(nheads / heads per block)
  // workspace
  float* hbuf;          // [batch, nchunks, dim, dstate]: state entering each chunk
  float* gbuf;          // [batch, nchunks, dim, dstate]: adjoint leaving each chunk
  float* dd_part;       // [batch, nchunks, dim]
  float* db_part;       // [batch, seqlen, ngroups, dstate]
  float* dc_part;       // [batch, seqlen, ngroups, dstate]
  float* da_part;       // [batch, nchunks, nheads]
};
constexpr int kSsdBwdHeadsPerBlock = 16;
hipError_t launch_ssd_bwd_mm(const SsdBwdArgs& a, hipStream_t stream);
bool ssd_supported(int64_t headdim, int64_t dstate);
hipError_t launch_ssd(const SsdArgs& a, int dstate, hipStream_t stream);

// Enqueue the seqlen == 0 case: h_last = h0 (or zeros).
hipError_t launch_copy_state(const float* h0, float* h_last, int64_t count,
                             hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, bool io_bf16, hipStream_t stream);

}  // namespace ssm
