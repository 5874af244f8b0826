// ssm_abi.cpp -- the extern "C" entry points declared in include/ssm.h:
// argument validation (entirely on the host, before any HIP call), the
// execution plan, workspace carving and dispatch to the kernels.

#include "ssm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "ssm_launch.h"

namespace {

constexpr int64_t kWave = 64;
constexpr int64_t kDState = 16;
// Design point of the schedule (MI355X: 256 CUs).  The scan's inner loop is
// bound by VALU issue, which needs several resident waves per SIMD: the plan
// keeps 4 waves per 64-channel group (4 states each; at most five such blocks
// fit a CU's LDS) and picks the chunk count K and the schedule with the cost
// model of plan_cost below.
constexpr int64_t kCUs = 256;
constexpr int64_t kResident = 5;     // main-pass blocks per CU (30 KB of LDS each)
constexpr int64_t kTargetBlocks = kResident * kCUs;
constexpr int64_t kMinChunk = 256;   // shortest chunk the plan will cut
// Longest chunk the plan leaves: long sequences with few channel groups get
// at least L / kMaxChunk chunks, so that blocks stay short enough to balance
// over the CUs (single sequence, L = 262144, D = 4096: 7.3 ms at 20 chunks,
// 6.6-6.9 ms at 64 to 256).
constexpr int64_t kMaxChunk = 2048;

bool valid_dtype(int t) { return t == SSM_DTYPE_F32 || t == SSM_DTYPE_BF16; }

constexpr int64_t kMaxGridYZ = 65535;  // HIP limit on grid.y and grid.z
// Batch rows per launch when a scan has more than kMaxGridYZ rows: a multiple
// of 8, so that every slice's tensor pointers keep 16-byte alignment.
constexpr int64_t kSliceRows = 65528;

// The kernels address one chunk of an [b, L, dim] tensor with 32-bit byte
// offsets; a chunk spans at most this many bytes.
constexpr int64_t kMaxChunkBytes = (int64_t)1 << 31;

// Chunk length for a request of `nchunks`: at least enough chunks that none
// exceeds kMaxChunkBytes, at most min(seqlen, grid limit); the length is
// rounded up to whole tiles (chunks start on a tile boundary).
int64_t chunk_length(int64_t seqlen, int64_t dim, int io_dtype, int64_t nchunks) {
  if (seqlen <= 0) return 1;
  const int64_t tile = ssm::scan_tile_steps();
  const int64_t row = std::max<int64_t>(1, dim) * (io_dtype == SSM_DTYPE_BF16 ? 2 : 4);
  const int64_t max_rows = std::max<int64_t>(tile, (kMaxChunkBytes / row) / tile * tile);
  nchunks = std::max<int64_t>(nchunks, (seqlen + max_rows - 1) / max_rows);
  const int64_t k = std::max<int64_t>(1, std::min<int64_t>({nchunks, seqlen, kMaxGridYZ}));
  const int64_t len = (seqlen + k - 1) / k;
  return (len + tile - 1) / tile * tile;
}

// Number of chunks of length chunk_length(...) covering the sequence.
int effective_chunks(int64_t seqlen, int64_t dim, int io_dtype, int64_t nchunks) {
  if (seqlen <= 0) return 1;
  const int64_t len = chunk_length(seqlen, dim, io_dtype, nchunks);
  return (int)((seqlen + len - 1) / len);
}

// Cost model of a chunk plan, in steps on the critical path (fitted to plan
// sweeps of three layer shapes on MI355X: batch 4 x 4096 x 5120, 8 x 2048 x
// 1536 and 1 x 262144 x 4096; it ranks first the fastest measured plan of
// each, at the first shape the one of two equally fast plans, K = 4 and 5,
// that reads less).  A launch of n equal blocks of `len` steps keeps its most loaded CU
// busy for r = ceil(n / 256) blocks, in rounds of kResident resident blocks;
// with fewer than kResident blocks on a CU (r < kResident, or the last round
// of a larger r) its VALU issue slots go partly idle (measured slow-down for
// 1 .. 4 resident blocks).  A pre-pass step (state only, from a zero state) costs kPre4 of a
// main-pass step in a 4-wave block (two-launch schedule, beside chunk 0's main
// pass; the wave-independent pre-pass) and kPre8 in the 8-wave blocks of the
// three-pass schedule.  Four resident blocks (4 waves per SIMD) issue as fast
// as five: at batch 4 x 4096 x 5120 the main pass ran 60.1 ns per block-step
// with four per CU against 59.5 with five.
constexpr double kPre4 = 0.71, kPre8 = 0.72;
// x and delta of every chunk that gets a pre-pass are read from HBM twice.
// The issue model does not see that traffic; each whole extra read of x and
// delta adds kReread to a plan's cost, so that of two plans it rates equal
// the one that moves fewer bytes wins (the traffic is HBM bandwidth taken
// from whatever else runs on the GPU).
constexpr double kReread = 0.01;

double launch_cost(int64_t nblocks, int64_t len, double weight) {
  static const double slow[kResident] = {1.6, 1.6, 1.25, 1.10, 1.0};
  const int64_t r = (nblocks + kCUs - 1) / kCUs;
  // rounds of kResident blocks, then a last round of `part` blocks that runs
  // at the lower occupancy
  const int64_t full = r / kResident, part = r % kResident;
  return (double)len * weight *
         ((double)(full * kResident) + (part ? (double)part * slow[part] : 0.0));
}

// Cost of K chunks of `len` steps for `groups` channel groups in the two
// schedules (see launch_scan: two-launch = chunk 0's main pass beside the
// pre-pass of chunks 1 .. K-2, then the main pass of chunks 1 .. K-1;
// three-pass = the pre-pass of chunks 0 .. K-2, then the main pass of all K).
void plan_cost(int64_t groups, int64_t len, int64_t k, double* two, double* three) {
  if (k <= 1) {
    *two = *three = launch_cost(groups, len, 1.0);
    return;
  }
  const int64_t nb = groups * (k - 1);
  const double kd = (double)k;
  *two = (launch_cost(nb, len, (1.0 + kPre4 * (double)(k - 2)) / (double)(k - 1)) +
          launch_cost(nb, len, 1.0)) *
         (1.0 + kReread * (kd - 2.0) / kd);
  *three = (launch_cost(nb, len, kPre8) + launch_cost(groups * k, len, 1.0)) *
           (1.0 + kReread * (kd - 1.0) / kd);
}

int64_t channel_groups(int64_t batch, int64_t dim) {
  return std::max<int64_t>(1, batch * ((dim + kWave - 1) / kWave));
}

// Schedule bits (0: two-launch, ssm::kPhaseThreePass) that the model prefers
// for K effective chunks.
int plan_schedule(int64_t batch, int64_t seqlen, int64_t dim, int io_dtype, int k) {
  if (k <= 1) return 0;
  double two, three;
  plan_cost(channel_groups(batch, dim), chunk_length(seqlen, dim, io_dtype, k), k, &two,
            &three);
  return three < two ? ssm::kPhaseThreePass : 0;
}

// Automatic plan: 4 waves per group of 64 channels; the chunk count is the
// cheapest under plan_cost among K from L / kMaxChunk up to about twice the
// count that gives the main pass kTargetBlocks blocks (chunks no shorter than
// kMinChunk unless L / kMaxChunk asks for it); between equal costs (within
// 0.2%) the larger K, whose shorter blocks balance better over the CUs.
void auto_plan(int64_t batch, int64_t seqlen, int64_t dim, int io_dtype, int* G, int* K) {
  *G = 4;
  const int64_t groups = channel_groups(batch, dim);
  const int64_t kt = (kTargetBlocks + groups / 2) / groups + 1;
  const int64_t kcap = std::max<int64_t>(1, seqlen / kMinChunk);
  const int64_t lo = std::max<int64_t>(1, (seqlen + kMaxChunk - 1) / kMaxChunk);
  const int64_t hi = std::max({lo, std::min(2 * kt, kcap), std::min(2 * lo, kcap)});
  const int64_t stride = std::max<int64_t>(1, (hi - lo) / 64);  // at most ~65 candidates
  int best_k = effective_chunks(seqlen, dim, io_dtype, lo);
  double best = -1.0;
  for (int64_t c = lo; c <= hi; c += stride) {
    const int k = effective_chunks(seqlen, dim, io_dtype, c);
    double two, three;
    plan_cost(groups, chunk_length(seqlen, dim, io_dtype, k), k, &two, &three);
    const double cost = std::min(two, three);
    if (best < 0.0 || cost <= best * 1.002) {
      if (best < 0.0 || cost < best) best = cost;
      best_k = k;
    }
  }
  *K = best_k;
}

size_t workspace_for(int64_t batch, int64_t dim, int K) {
  return ssm::scan_workspace_layout(batch, dim, K).total;
}

bool sizes_ok(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  return batch >= 0 && seqlen >= 0 && dim >= 0 && dstate > 0 &&
         dim <= (int64_t)INT32_MAX && batch <= (int64_t)INT32_MAX;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_HIP; }

// Scratch of ssm_scan_fwd_noalloc: the chunk-carry workspace (per-chunk end
// states, entering states and delta sums) lives in this file-scope device
// array instead of a caller buffer.  Every GPU the library runs on holds its
// own copy at its own address until the process ends.  In host code the name
// `scratch` is a host-side stand-in, not a device address: kernels get the
// address hipGetSymbolAddress returns for the device, looked up once per
// device (with that device current) and kept in scratch_ptr.
__device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
void* scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// Device address of `scratch` on the device that runs `stream`.
int scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  const hipError_t e0 = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e0 != hipSuccess) return SSM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SSM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SSM_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return SSM_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return SSM_ERR_HIP;
    if (e != hipSuccess || !p) return SSM_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return SSM_OK;
}

// Every tensor pointer must be 16-byte aligned (the kernels use 16-byte
// vector and 4-byte scalar accesses on these bases).
bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
template <typename... P> bool all_aligned(P... p) { return (aligned(p) && ...); }

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_str(int status) {
  switch (status) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_INVALID_ARG: return "SSM_ERR_INVALID_ARG: invalid argument";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: no kernel for this request";
    case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE: workspace missing or too small";
    case SSM_ERR_HIP: return "SSM_ERR_HIP: HIP runtime or launch failure";
  }
  return "SSM_ERR_UNKNOWN: unknown status code";
}

int ssm_scan_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                  int* waves_per_group, int* nchunks, int* phase) {
  if (!waves_per_group || !nchunks || !sizes_ok(batch, seqlen, dim, dstate) ||
      !valid_dtype(io_dtype))
    return SSM_ERR_INVALID_ARG;
  auto_plan(batch, seqlen, dim, io_dtype, waves_per_group, nchunks);
  *nchunks = effective_chunks(seqlen, dim, io_dtype, *nchunks);
  if (phase) *phase = 3 | plan_schedule(batch, seqlen, dim, io_dtype, *nchunks);
  return SSM_OK;
}

int64_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                 int io_dtype, int nchunks) {
  if (!sizes_ok(batch, seqlen, dim, dstate) || !valid_dtype(io_dtype)) return -1;
  if (nchunks <= 0) {
    int g;
    auto_plan(batch, seqlen, dim, io_dtype, &g, &nchunks);
  }
  if (batch == 0 || dim == 0 || seqlen == 0) return 0;
  if (dstate != kDState) return 0;  // wide states: one pass, no carry workspace
  nchunks = effective_chunks(seqlen, dim, io_dtype, nchunks);
  return (int64_t)workspace_for(batch, dim, nchunks);
}

}  // extern "C"

namespace {

// Validation and launch shared by the plain and the fused scan.  With
// pro.d_conv > 0, x and delta are x_raw and delta_raw.
int scan_entry(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
               const void* x, const void* delta, const float* A, const void* B, const void* C,
               const float* Dskip, const void* z, const float* h0, void* y, float* h_last,
               void* workspace, size_t workspace_bytes, int waves_per_group, int nchunks,
               int phase, void* stream, const ssm::Prologue& pro, int a_per_channel = 0,
               int euler = 0, bool use_scratch = false) {
  if (!sizes_ok(batch, seqlen, dim, dstate) || !valid_dtype(io_dtype))
    return SSM_ERR_INVALID_ARG;
  // phase: bits 1 and 2 select the launches, bit 4 the three-pass schedule;
  // 0 = both launches in the schedule plan_schedule prefers
  const bool auto_schedule = phase == 0;
  if (auto_schedule) phase = 3;
  if (phase < 1 || phase > 7 || (phase & 3) == 0) return SSM_ERR_INVALID_ARG;
  if (batch == 0 || dim == 0) return SSM_OK;
  // state sizes other than 16 run the one-pass wide-state kernels: no chunk
  // plan, no fused prologue, one call
  const bool wide = dstate != kDState;
  if (wide && !ssm::scan_wide_supported(dstate)) return SSM_ERR_UNSUPPORTED;
  if (wide && (pro.d_conv > 0 || (phase & 3) != 3)) return SSM_ERR_UNSUPPORTED;
  if (!A) return SSM_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (seqlen == 0) {
    if (!h_last || !(phase & 2)) return SSM_OK;
    if ((const void*)h_last == (const void*)h0 || (const void*)h_last == (const void*)A)
      return SSM_ERR_INVALID_ARG;
    if (!all_aligned(h0, h_last)) return SSM_ERR_INVALID_ARG;
    return hip_status(ssm::launch_copy_state(h0, h_last, batch * dim * dstate, s));
  }
  if (!x || !delta || !B || !C || !y) return SSM_ERR_INVALID_ARG;
  // outputs must not alias any input
  const void* ins[] = {x, delta, A, B, C, Dskip, z, h0, pro.conv_w, pro.conv_b, pro.delta_bias};
  for (const void* in : ins) {
    if (!in) continue;
    if (in == y || in == (const void*)h_last) return SSM_ERR_INVALID_ARG;
  }
  if ((const void*)h_last == y) return SSM_ERR_INVALID_ARG;
  if (!all_aligned(x, delta, A, B, C, Dskip, z, h0, y, h_last, workspace) ||
      !all_aligned(pro.conv_w, pro.conv_b, pro.delta_bias))
    return SSM_ERR_INVALID_ARG;
  if (batch > kMaxGridYZ) {
    // The kernels put batch rows on grid.y (at most 65535): run slices of
    // kSliceRows rows in order on the stream.  Rows are independent and the
    // workspace, sized for the whole batch, is reused slice by slice, which
    // is why the two phases cannot be enqueued apart here.
    if ((phase & 3) != 3) return SSM_ERR_UNSUPPORTED;
    const int64_t io = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
    const int64_t xrow = seqlen * dim * io, bcrow = seqlen * dstate * io, srow = dim * dstate * 4;
    for (int64_t r0 = 0; r0 < batch; r0 += kSliceRows) {
      auto at = [r0](const void* p, int64_t per_row) -> const char* {
        return p ? static_cast<const char*>(p) + r0 * per_row : nullptr;
      };
      const int st = scan_entry(
          std::min(kSliceRows, batch - r0), seqlen, dim, dstate, io_dtype, at(x, xrow),
          at(delta, xrow), A, at(B, bcrow), at(C, bcrow), Dskip, at(z, xrow),
          reinterpret_cast<const float*>(at(h0, srow)), const_cast<char*>(at(y, xrow)),
          reinterpret_cast<float*>(const_cast<char*>(at(h_last, srow))), workspace,
          workspace_bytes, waves_per_group, nchunks, auto_schedule ? 0 : phase, stream, pro,
          a_per_channel, euler, use_scratch);
      if (st != SSM_OK) return st;
    }
    return SSM_OK;
  }
  if (wide) {
    ssm::ScanArgs a{};
    a.x = x;
    a.delta = delta;
    a.A = A;
    a.B = B;
    a.C = C;
    a.Dskip = Dskip;
    a.z = z;
    a.h0 = h0;
    a.y = y;
    a.h_last = h_last;
    a.seqlen = seqlen;
    a.chunk_len = seqlen;
    a.nchunks = 1;
    a.dim = (int)dim;
    a.batch = (int)batch;
    a.a_per_channel = a_per_channel;
    a.euler = euler;
    return hip_status(ssm::launch_scan_wide(a, (int)dstate, io_dtype == SSM_DTYPE_BF16, s));
  }

  int G = 0, K = 0;
  auto_plan(batch, seqlen, dim, io_dtype, &G, &K);
  if (waves_per_group > 0) G = waves_per_group;
  if (nchunks > 0) K = nchunks;
  if (G != 2 && G != 4 && G != 8 && G != 16) return SSM_ERR_UNSUPPORTED;
  if (pro.d_conv > 0 && G == 16) return SSM_ERR_UNSUPPORTED;  // fused loader: G <= 8
  if ((a_per_channel || euler) && G == 16) return SSM_ERR_UNSUPPORTED;  // variants: G <= 8
  const int64_t chunk_len = chunk_length(seqlen, dim, io_dtype, K);
  K = effective_chunks(seqlen, dim, io_dtype, K);  // == ceil(seqlen / chunk_len)
  if (auto_schedule) phase |= plan_schedule(batch, seqlen, dim, io_dtype, K);

  const ssm::ScanWorkspace ws = ssm::scan_workspace_layout(batch, dim, K);
  if (use_scratch && ws.total > 0) {
    // the file-scope scratch instead of a caller buffer (after every
    // argument check: nothing before this point touches the GPU)
    if (ws.total > workspace_bytes) return SSM_ERR_WORKSPACE;
    const int st = scratch_for_stream(s, &workspace);
    if (st != SSM_OK) return st;
  }
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return SSM_ERR_WORKSPACE;
  if (ws.total > 0) {
    for (const void* in : ins)
      if (in && in == workspace) return SSM_ERR_INVALID_ARG;
    if (workspace == y || workspace == (void*)h_last) return SSM_ERR_INVALID_ARG;
  }

  ssm::ScanArgs a{};
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = Dskip;
  a.z = z;
  a.h0 = h0;
  a.y = y;
  a.h_last = h_last;
  char* wsb = static_cast<char*>(workspace);
  a.ws_hloc = K > 1 ? reinterpret_cast<float*>(wsb + ws.hloc_off) : nullptr;
  a.ws_hin = K > 1 ? reinterpret_cast<float*>(wsb + ws.hin_off) : nullptr;
  a.ws_sdelta = K > 1 ? reinterpret_cast<double*>(wsb + ws.sdelta_off) : nullptr;
  a.seqlen = seqlen;
  a.chunk_len = chunk_len;
  a.nchunks = K;
  a.dim = (int)dim;
  a.batch = (int)batch;
  a.pro = pro;
  a.a_per_channel = a_per_channel;
  a.euler = euler;
  return hip_status(ssm::launch_scan(a, io_dtype == SSM_DTYPE_BF16, G, phase, s));
}

}  // namespace

extern "C" {

int ssm_scan_fwd_phase(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                       int io_dtype, const void* x, const void* delta, const float* A,
                       const void* B, const void* C, const float* Dskip, const void* z,
                       const float* h0, void* y, float* h_last, void* workspace,
                       size_t workspace_bytes, int waves_per_group, int nchunks, int phase,
                       void* stream) {
  if (phase < 1) return SSM_ERR_INVALID_ARG;
  const ssm::Prologue none{};
  return scan_entry(batch, seqlen, dim, dstate, io_dtype, x, delta, A, B, C, Dskip, z, h0, y,
                    h_last, workspace, workspace_bytes, waves_per_group, nchunks, phase, stream,
                    none);
}

int ssm_scan_fwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                    const void* x, const void* delta, const float* A, int a_per_channel,
                    int discretization, const void* B, const void* C, const float* Dskip,
                    const void* z, const float* h0, void* y, float* h_last, void* workspace,
                    size_t workspace_bytes, int waves_per_group, int nchunks, void* stream) {
  if (a_per_channel != 0 && a_per_channel != 1) return SSM_ERR_INVALID_ARG;
  if (discretization != SSM_DISC_ZOH && discretization != SSM_DISC_EULER)
    return SSM_ERR_INVALID_ARG;
  const ssm::Prologue none{};
  return scan_entry(batch, seqlen, dim, dstate, io_dtype, x, delta, A, B, C, Dskip, z, h0, y,
                    h_last, workspace, workspace_bytes, waves_per_group, nchunks, 0, stream,
                    none, a_per_channel, discretization == SSM_DISC_EULER ? 1 : 0);
}

int ssm_scan_fwd_fused(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                       int io_dtype, const void* x_raw, const float* conv_w,
                       const float* conv_b, int d_conv, int conv_silu, const void* delta_raw,
                       const float* delta_bias, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, const float* h0, void* y,
                       float* h_last, void* workspace, size_t workspace_bytes,
                       int waves_per_group, int nchunks, void* stream) {
  if (d_conv < 1 || (conv_silu != 0 && conv_silu != 1)) return SSM_ERR_INVALID_ARG;
  if (!sizes_ok(batch, seqlen, dim, dstate) || !valid_dtype(io_dtype))
    return SSM_ERR_INVALID_ARG;
  if (batch > 0 && dim > 0 && seqlen > 0 && !conv_w) return SSM_ERR_INVALID_ARG;
  if (d_conv > 4) return SSM_ERR_UNSUPPORTED;
  ssm::Prologue pro{};
  pro.conv_w = conv_w;
  pro.conv_b = conv_b;
  pro.delta_bias = delta_bias;
  pro.d_conv = d_conv;
  pro.conv_silu = conv_silu;
  return scan_entry(batch, seqlen, dim, dstate, io_dtype, x_raw, delta_raw, A, B, C, Dskip, z,
                    h0, y, h_last, workspace, workspace_bytes, waves_per_group, nchunks, 0,
                    stream, pro);
}

int ssm_scan_fwd_planned(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         int io_dtype, const void* x, const void* delta, const float* A,
                         const void* B, const void* C, const float* Dskip, const void* z,
                         const float* h0, void* y, float* h_last, void* workspace,
                         size_t workspace_bytes, int waves_per_group, int nchunks,
                         void* stream) {
  const ssm::Prologue none{};
  return scan_entry(batch, seqlen, dim, dstate, io_dtype, x, delta, A, B, C, Dskip, z, h0, y,
                    h_last, workspace, workspace_bytes, waves_per_group, nchunks, 0, stream,
                    none);
}

int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 const void* x, const void* delta, const float* A, const void* B,
                 const void* C, const float* Dskip, const void* z, const float* h0, void* y,
                 float* h_last, void* workspace, size_t workspace_bytes, void* stream) {
  return ssm_scan_fwd_planned(batch, seqlen, dim, dstate, io_dtype, x, delta, A, B, C, Dskip,
                              z, h0, y, h_last, workspace, workspace_bytes, 0, 0, stream);
}

int ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         int io_dtype, const void* x, const void* delta, const float* A,
                         const void* B, const void* C, const float* Dskip, const void* z,
                         const float* h0, void* y, float* h_last, int waves_per_group,
                         int nchunks, void* stream) {
  const ssm::Prologue none{};
  return scan_entry(batch, seqlen, dim, dstate, io_dtype, x, delta, A, B, C, Dskip, z, h0, y,
                    h_last, nullptr, SSM_NOALLOC_SCRATCH_BYTES, waves_per_group, nchunks, 0,
                    stream, none, 0, 0, true);
}

int ssm_decode_step_ex(int64_t batch, int64_t dim, int64_t dstate, int io_dtype, float* h,
                       const void* x, const void* delta, const float* A, int a_per_channel,
                       int discretization, const void* B, const void* C, const float* Dskip,
                       const void* z, void* y, void* stream) {
  if (a_per_channel != 0 && a_per_channel != 1) return SSM_ERR_INVALID_ARG;
  if (discretization != SSM_DISC_ZOH && discretization != SSM_DISC_EULER)
    return SSM_ERR_INVALID_ARG;
  if (!sizes_ok(batch, 1, dim, dstate) || !valid_dtype(io_dtype)) return SSM_ERR_INVALID_ARG;
  if (batch == 0 || dim == 0) return SSM_OK;
  if (dstate != kDState && !ssm::scan_wide_supported(dstate)) return SSM_ERR_UNSUPPORTED;
  if (batch * dim * (dstate / 4) / 256 >= (int64_t)UINT32_MAX) return SSM_ERR_UNSUPPORTED;
  if (!h || !x || !delta || !A || !B || !C || !y) return SSM_ERR_INVALID_ARG;
  const void* ins[] = {x, delta, A, B, C, Dskip, z};
  for (const void* in : ins)
    if (in && (in == y || in == (const void*)h)) return SSM_ERR_INVALID_ARG;
  if ((const void*)h == y) return SSM_ERR_INVALID_ARG;
  if (!all_aligned(h, x, delta, A, B, C, Dskip, z, y)) return SSM_ERR_INVALID_ARG;
  ssm::DecodeArgs a{};
  a.h = h;
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = Dskip;
  a.z = z;
  a.y = y;
  a.batch = batch;
  a.dim = (int)dim;
  a.dstate = (int)dstate;
  a.a_per_channel = a_per_channel;
  a.euler = discretization == SSM_DISC_EULER ? 1 : 0;
  return hip_status(ssm::launch_decode(a, io_dtype == SSM_DTYPE_BF16,
                                       static_cast<hipStream_t>(stream)));
}

int ssm_decode_step(int64_t batch, int64_t dim, int64_t dstate, int io_dtype, float* h,
                    const void* x, const void* delta, const float* A, const void* B,
                    const void* C, const float* Dskip, const void* z, void* y,
                    void* stream) {
  return ssm_decode_step_ex(batch, dim, dstate, io_dtype, h, x, delta, A, 0, SSM_DISC_ZOH, B,
                            C, Dskip, z, y, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward of the scan
// ---------------------------------------------------------------------------
namespace {

// Sequence segments of the per-head scan.  With at least kSsdFullBlocks
// blocks (2.5 per CU) none; with fewer, enough for about kSsdSplitBlocks,
// none shorter than kSsdMinSeg steps.  nsplit > 0 asks for that many.
// Segments are whole chunks of ssm::kSsdChunk steps.  Returns the number of
// segments and their length.
constexpr int64_t kSsdFullBlocks = 640;
constexpr int64_t kSsdSplitBlocks = 1280;
constexpr int64_t kSsdMinSeg = 256;
int ssd_plan(int64_t batch, int64_t seqlen, int64_t nheads, int nsplit, int64_t* seg_len) {
  constexpr int64_t Q = ssm::kSsdChunk;
  int64_t k = nsplit;
  if (k <= 0) {
    const int64_t blocks = std::max<int64_t>(1, 2 * nheads * batch);
    k = blocks >= kSsdFullBlocks ? 1 : (kSsdSplitBlocks + blocks - 1) / blocks;
    k = std::min<int64_t>(k, std::max<int64_t>(1, seqlen / kSsdMinSeg));
  }
  k = std::max<int64_t>(1, std::min<int64_t>({k, (seqlen + Q - 1) / Q, kMaxGridYZ}));
  int64_t len = (seqlen + k - 1) / k;
  len = std::max<int64_t>(Q, (len + Q - 1) / Q * Q);
  *seg_len = len;
  return (int)std::max<int64_t>(1, (seqlen + len - 1) / len);
}

// Workspace pointers of a backward (chunk carries and partial sums).
void set_bwd_workspace(ssm::BwdArgs& a, const ssm::BwdWorkspace& w, char* base, int K) {
  if (K > 1) {
    a.f.ws_hloc = reinterpret_cast<float*>(base + w.fwd.hloc_off);
    a.f.ws_hin = reinterpret_cast<float*>(base + w.fwd.hin_off);
    a.f.ws_sdelta = reinterpret_cast<double*>(base + w.fwd.sdelta_off);
    a.ws_eloc = reinterpret_cast<float*>(base + w.rev_base + w.rev.hloc_off);
    a.ws_ein = reinterpret_cast<float*>(base + w.rev_base + w.rev.hin_off);
    a.ws_sdr = reinterpret_cast<double*>(base + w.rev_base + w.rev.sdelta_off);
  }
  a.ws_pdB = reinterpret_cast<float*>(base + w.pdB_off);
  a.ws_pdC = reinterpret_cast<float*>(base + w.pdC_off);
  a.ws_pdA = reinterpret_cast<float*>(base + w.pdA_off);
  a.ws_pdD = reinterpret_cast<float*>(base + w.pdD_off);
}

// Workspace of the per-head backward: the sliced backward's, plus delta and A
// repeated over each head's channels, the per-channel dA and (unused
// afterwards) per-channel ddelta.
struct SsdBwdLayout {
  ssm::BwdSliceWorkspace s;
  size_t delta_off, ach_off, dach_off, ddch_off, total;
};
SsdBwdLayout ssd_bwd_layout(int64_t batch, int64_t seqlen, int64_t dim, int K, int io_bytes) {
  auto align = [](size_t v) { return (v + 255) & ~size_t(255); };
  SsdBwdLayout l{};
  l.s = ssm::bwd_slice_layout(batch, seqlen, dim, K, io_bytes);
  const size_t rows = (size_t)batch * seqlen * dim * io_bytes;
  l.delta_off = align(l.s.total);
  l.ach_off = l.delta_off + align(rows);
  l.dach_off = l.ach_off + align((size_t)dim * sizeof(float));
  l.ddch_off = l.dach_off + align((size_t)dim * sizeof(float));
  l.total = l.ddch_off + align(rows);
  return l;
}

// The masked-matrix backward (chunk-parallel, matrix cores): bf16 I/O,
// 64-channel heads, 64 or 128 states, at most kMaxGridYZ chunks of 32 steps;
// other shapes take the recurrence kernels with dt repeated over channels.
bool ssd_bwd_mm(int io_dtype, int64_t headdim, int64_t dstate, int64_t seqlen) {
  return io_dtype == SSM_DTYPE_BF16 && ssm::ssd_supported(headdim, dstate) &&
         (seqlen + 31) / 32 <= kMaxGridYZ;
}

struct SsdBwdMmLayout {
  size_t hbuf, gbuf, dd, db, dc, da, dh0, total;
  int nchunks, ngroups;
};
SsdBwdMmLayout ssd_bwd_mm_layout(int64_t batch, int64_t seqlen, int64_t nheads, int64_t dim,
                                 int64_t dstate) {
  auto align = [](size_t v) { return (v + 255) & ~size_t(255); };
  SsdBwdMmLayout l{};
  l.nchunks = (int)((seqlen + 31) / 32);
  l.ngroups = (int)((nheads + ssm::kSsdBwdHeadsPerBlock - 1) / ssm::kSsdBwdHeadsPerBlock);
  const size_t K = (size_t)l.nchunks, f = sizeof(float);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align(bytes);
    return at;
  };
  l.hbuf = take((size_t)batch * K * dim * dstate * f);
  l.gbuf = take((size_t)batch * K * dim * dstate * f);
  l.dd = take((size_t)batch * K * dim * f);
  l.db = take((size_t)batch * seqlen * l.ngroups * dstate * f);
  l.dc = take((size_t)batch * seqlen * l.ngroups * dstate * f);
  l.da = take((size_t)batch * K * nheads * f);
  l.dh0 = take((size_t)batch * dim * dstate * f);
  l.total = o;
  return l;
}

// State sizes whose backward runs as 16-state slices.
bool bwd_sliced(int64_t dstate) { return dstate == 32 || dstate == 64 || dstate == 128; }

// Chunk length and count of the backward plan: chunks of at most
// ssm::kBwdChunk steps, starting on tile boundaries.
void bwd_plan(int64_t seqlen, int64_t* chunk_len, int* nchunks) {
  const int64_t tile = ssm::scan_tile_steps();
  const int64_t k = std::max<int64_t>(1, (seqlen + ssm::kBwdChunk - 1) / ssm::kBwdChunk);
  int64_t len = std::max<int64_t>(1, (seqlen + k - 1) / k);
  len = (len + tile - 1) / tile * tile;
  *chunk_len = len;
  *nchunks = (int)std::max<int64_t>(1, (seqlen + len - 1) / len);
}

}  // namespace

extern "C" {

int64_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim,
                                     int64_t dstate, int io_dtype) {
  if (!sizes_ok(batch, seqlen, dim, dstate) || !valid_dtype(io_dtype)) return -1;
  if (batch == 0 || dim == 0 || seqlen == 0) return 0;
  int64_t len;
  int K;
  bwd_plan(seqlen, &len, &K);
  if (bwd_sliced(dstate))
    return (int64_t)ssm::bwd_slice_layout(batch, seqlen, dim, K,
                                          io_dtype == SSM_DTYPE_BF16 ? 2 : 4).total;
  return (int64_t)ssm::bwd_workspace_layout(batch, seqlen, dim, K).total;
}

int ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 const void* x, const void* delta, const float* A, int a_per_channel,
                 int discretization, const void* B, const void* C, const float* Dskip,
                 const void* z, const float* h0, const void* dy, const float* dh_last,
                 void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                 float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  if (!sizes_ok(batch, seqlen, dim, dstate) || !valid_dtype(io_dtype)) return SSM_ERR_INVALID_ARG;
  if (a_per_channel != 0 && a_per_channel != 1) return SSM_ERR_INVALID_ARG;
  if (discretization != SSM_DISC_ZOH && discretization != SSM_DISC_EULER)
    return SSM_ERR_INVALID_ARG;
  if (dstate != kDState && !bwd_sliced(dstate)) return SSM_ERR_UNSUPPORTED;
  if (!A || !dA) return SSM_ERR_INVALID_ARG;
  if ((z == nullptr) != (dz == nullptr)) return SSM_ERR_INVALID_ARG;
  if (seqlen > 0 && batch > 0 && dim > 0 &&
      (!x || !delta || !B || !C || !dy || !dx || !ddelta || !dB || !dC))
    return SSM_ERR_INVALID_ARG;
  const void* ins[] = {x, delta, A, B, C, Dskip, z, h0, dy, dh_last};
  const void* outs[] = {dx, ddelta, dA, dB, dC, dD, dz, dh0};
  for (const void* o : outs) {
    if (!o) continue;
    for (const void* in : ins)
      if (in == o) return SSM_ERR_INVALID_ARG;
    int same = 0;
    for (const void* o2 : outs) same += (o2 == o);
    if (same > 1) return SSM_ERR_INVALID_ARG;
  }
  if (!all_aligned(x, delta, A, B, C, Dskip, z, h0, dy, dh_last, workspace) ||
      !all_aligned(dx, ddelta, dA, dB, dC, dD, dz, dh0))
    return SSM_ERR_INVALID_ARG;
  if (batch > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  auto s = static_cast<hipStream_t>(stream);
  if (dim == 0) return SSM_OK;
  const int64_t na = a_per_channel ? dim : dim * dstate;
  if (batch == 0 || seqlen == 0) {
    // no steps: dA = dD = 0, dh0 = dh_last (or 0)
    hipError_t e = ssm::launch_copy_state(nullptr, dA, na, s);
    if (e == hipSuccess && dD) e = ssm::launch_copy_state(nullptr, dD, dim, s);
    if (e == hipSuccess && dh0 && batch > 0)
      e = ssm::launch_copy_state(dh_last, dh0, batch * dim * dstate, s);
    return hip_status(e);
  }
  int64_t chunk_len;
  int K;
  bwd_plan(seqlen, &chunk_len, &K);
  if (K > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  const bool sliced = dstate != kDState;
  const ssm::BwdSliceWorkspace ws =
      ssm::bwd_slice_layout(batch, seqlen, dim, K, io_dtype == SSM_DTYPE_BF16 ? 2 : 4);
  const ssm::BwdWorkspace& w = ws.base;
  if (!workspace || workspace_bytes < (sliced ? ws.total : w.total)) return SSM_ERR_WORKSPACE;
  for (const void* in : ins)
    if (in && in == workspace) return SSM_ERR_INVALID_ARG;
  for (const void* o : outs)
    if (o && o == workspace) return SSM_ERR_INVALID_ARG;

  char* base = static_cast<char*>(workspace);
  ssm::BwdArgs a{};
  set_bwd_workspace(a, w, base, K);
  ssm::ScanArgs& f = a.f;
  f.x = x;
  f.delta = delta;
  f.A = A;
  f.B = B;
  f.C = C;
  f.Dskip = Dskip;
  f.z = z;
  f.h0 = h0;
  f.seqlen = seqlen;
  f.chunk_len = chunk_len;
  f.dim = (int)dim;
  f.batch = (int)batch;
  f.nchunks = K;
  f.a_per_channel = a_per_channel;
  f.euler = discretization == SSM_DISC_EULER ? 1 : 0;
  a.dy = dy;
  a.dh_last = dh_last;
  a.dx = dx;
  a.ddelta = ddelta;
  a.dz = dz;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dD = dD;
  a.dh0 = dh0;
  if (sliced)
    return hip_status(
        ssm::launch_scan_bwd_sliced(a, (int)dstate, io_dtype == SSM_DTYPE_BF16, base, ws, s));
  return hip_status(ssm::launch_scan_bwd(a, io_dtype == SSM_DTYPE_BF16, s));
}

int ssm_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                int io_dtype, int discretization, const void* x, const void* dt, const float* A,
                const void* B, const void* C, const float* Dskip, const void* z,
                const float* h0, void* y, float* h_last, void* workspace,
                size_t workspace_bytes, void* stream) {
  return ssm_ssd_fwd_planned(batch, seqlen, nheads, headdim, dstate, io_dtype, discretization, x,
                             dt, A, B, C, Dskip, z, h0, y, h_last, 1, workspace, workspace_bytes,
                             stream);
}

int64_t ssm_ssd_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                    int64_t headdim, int64_t dstate, int nsplit) {
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim <= 0 || dstate <= 0 ||
      nheads > (int64_t)INT32_MAX / headdim)
    return -1;
  if (batch == 0 || seqlen == 0 || nheads == 0) return 0;
  int64_t len;
  const int K = ssd_plan(batch, seqlen, nheads, nsplit, &len);
  return (int64_t)ssm::ssd_layout(batch, seqlen, nheads * headdim, nheads, dstate, K).total;
}

int ssm_ssd_fwd_planned(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate, int io_dtype, int discretization, const void* x,
                        const void* dt, const float* A, const void* B, const void* C,
                        const float* Dskip, const void* z, const float* h0, void* y,
                        float* h_last, int nsplit, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim <= 0 || dstate <= 0 ||
      !valid_dtype(io_dtype))
    return SSM_ERR_INVALID_ARG;
  if (discretization != SSM_DISC_ZOH && discretization != SSM_DISC_EULER)
    return SSM_ERR_INVALID_ARG;
  // the kernel addresses one 64-step chunk of a [b, L, dim] tensor with
  // 32-bit byte offsets: 64 * dim * 2 bytes must stay below 2^31
  if (nheads > ((int64_t)1 << 24) / headdim) return SSM_ERR_UNSUPPORTED;
  if (io_dtype != SSM_DTYPE_BF16 || !ssm::ssd_supported(headdim, dstate))
    return SSM_ERR_UNSUPPORTED;
  if (batch == 0 || nheads == 0) return SSM_OK;
  if (!A) return SSM_ERR_INVALID_ARG;
  const int64_t dim = nheads * headdim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (seqlen == 0) {
    if (!h_last) return SSM_OK;
    if ((const void*)h_last == (const void*)h0 || (const void*)h_last == (const void*)A)
      return SSM_ERR_INVALID_ARG;
    if (!all_aligned(h0, h_last)) return SSM_ERR_INVALID_ARG;
    return hip_status(ssm::launch_copy_state(h0, h_last, batch * dim * dstate, s));
  }
  if (!x || !dt || !B || !C || !y) return SSM_ERR_INVALID_ARG;
  const void* ins[] = {x, dt, A, B, C, Dskip, z, h0};
  for (const void* in : ins) {
    if (!in) continue;
    if (in == y || in == (const void*)h_last) return SSM_ERR_INVALID_ARG;
  }
  if ((const void*)h_last == y) return SSM_ERR_INVALID_ARG;
  if (!all_aligned(x, dt, A, B, C, Dskip, z, h0, y, h_last, workspace))
    return SSM_ERR_INVALID_ARG;
  int64_t seg_len;
  const int K = ssd_plan(batch, seqlen, nheads, nsplit, &seg_len);
  const ssm::SsdLayout l = ssm::ssd_layout(batch, seqlen, dim, nheads, dstate, K);
  if (!workspace || workspace_bytes < l.total) return SSM_ERR_WORKSPACE;
  for (const void* in : ins)
    if (in && in == workspace) return SSM_ERR_INVALID_ARG;
  if (workspace == y || workspace == (void*)h_last) return SSM_ERR_INVALID_ARG;
  char* base = static_cast<char*>(workspace);
  ssm::SsdArgs a{};
  a.nck = (seqlen + ssm::kSsdChunk - 1) / ssm::kSsdChunk;
  a.ws_cp = base + l.cp_off;
  a.ws_bt = base + l.bt_off;
  a.ws_mt = reinterpret_cast<float*>(base + l.mt_off);
  a.nseg = K;
  a.seg_len = seg_len;
  if (K > 1) {
    a.ws_hloc = reinterpret_cast<float*>(base + l.hloc_off);
    a.ws_hin = reinterpret_cast<float*>(base + l.hin_off);
    a.ws_dlog = reinterpret_cast<float*>(base + l.dlog_off);
  }
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = Dskip;
  a.z = z;
  a.h0 = h0;
  a.y = y;
  a.h_last = h_last;
  a.seqlen = seqlen;
  a.batch = batch;
  a.nheads = (int)nheads;
  a.dim = (int)dim;
  a.euler = discretization == SSM_DISC_EULER ? 1 : 0;
  return hip_status(ssm::launch_ssd(a, (int)dstate, s));
}

int64_t ssm_ssd_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads,
                                    int64_t headdim, int64_t dstate, int io_dtype) {
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim <= 0 || dstate <= 0 ||
      !valid_dtype(io_dtype) || nheads > (int64_t)INT32_MAX / headdim)
    return -1;
  if (batch == 0 || seqlen == 0 || nheads == 0) return 0;
  if (ssd_bwd_mm(io_dtype, headdim, dstate, seqlen))
    return (int64_t)ssd_bwd_mm_layout(batch, seqlen, nheads, nheads * headdim, dstate).total;
  int64_t len;
  int K;
  bwd_plan(seqlen, &len, &K);
  return (int64_t)ssd_bwd_layout(batch, seqlen, nheads * headdim, K,
                                 io_dtype == SSM_DTYPE_BF16 ? 2 : 4)
      .total;
}

int ssm_ssd_bwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                int io_dtype, int discretization, const void* x, const void* dt, const float* A,
                const void* B, const void* C, const float* Dskip, const void* z,
                const float* h0, const void* dy, const float* dh_last, void* dx, void* ddt,
                float* dA, void* dB, void* dC, float* dD, void* dz, float* dh0,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim <= 0 || dstate <= 0 ||
      !valid_dtype(io_dtype) || nheads > (int64_t)INT32_MAX / headdim)
    return SSM_ERR_INVALID_ARG;
  if (discretization != SSM_DISC_ZOH && discretization != SSM_DISC_EULER)
    return SSM_ERR_INVALID_ARG;
  if (dstate != kDState && !bwd_sliced(dstate)) return SSM_ERR_UNSUPPORTED;
  if (!A || !dA) return SSM_ERR_INVALID_ARG;
  if ((z == nullptr) != (dz == nullptr)) return SSM_ERR_INVALID_ARG;
  const int64_t dim = nheads * headdim;
  if (seqlen > 0 && batch > 0 && dim > 0 &&
      (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC))
    return SSM_ERR_INVALID_ARG;
  const void* ins[] = {x, dt, A, B, C, Dskip, z, h0, dy, dh_last};
  const void* outs[] = {dx, ddt, dA, dB, dC, dD, dz, dh0};
  for (const void* o : outs) {
    if (!o) continue;
    for (const void* in : ins)
      if (in == o) return SSM_ERR_INVALID_ARG;
    int same = 0;
    for (const void* o2 : outs) same += (o2 == o);
    if (same > 1) return SSM_ERR_INVALID_ARG;
  }
  if (!all_aligned(x, dt, A, B, C, Dskip, z, h0, dy, dh_last, workspace) ||
      !all_aligned(dx, ddt, dA, dB, dC, dD, dz, dh0))
    return SSM_ERR_INVALID_ARG;
  if (batch > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  auto s = static_cast<hipStream_t>(stream);
  if (dim == 0) return SSM_OK;
  if (batch == 0 || seqlen == 0) {
    // no steps: dA = dD = 0, dh0 = dh_last (or 0)
    hipError_t e = ssm::launch_copy_state(nullptr, dA, nheads, s);
    if (e == hipSuccess && dD) e = ssm::launch_copy_state(nullptr, dD, dim, s);
    if (e == hipSuccess && dh0 && batch > 0)
      e = ssm::launch_copy_state(dh_last, dh0, batch * dim * dstate, s);
    return hip_status(e);
  }
  if (ssd_bwd_mm(io_dtype, headdim, dstate, seqlen)) {
    // the kernels address one 32-step chunk of a [b, L, dim] tensor with
    // 32-bit byte offsets
    if (nheads > ((int64_t)1 << 24) / headdim) return SSM_ERR_UNSUPPORTED;
    const SsdBwdMmLayout l = ssd_bwd_mm_layout(batch, seqlen, nheads, dim, dstate);
    if (!workspace || workspace_bytes < l.total) return SSM_ERR_WORKSPACE;
    for (const void* p : ins)
      if (p && p == workspace) return SSM_ERR_INVALID_ARG;
    for (const void* o : outs)
      if (o && o == workspace) return SSM_ERR_INVALID_ARG;
    char* base = static_cast<char*>(workspace);
    auto fp = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
    ssm::SsdBwdArgs a{};
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.B = B;
    a.C = C;
    a.Dskip = Dskip;
    a.z = z;
    a.h0 = h0;
    a.dy = dy;
    a.dh_last = dh_last;
    a.dx = dx;
    a.ddt = ddt;
    a.dA = dA;
    a.dB = dB;
    a.dC = dC;
    a.dD = dD;
    a.dz = dz;
    a.dh0 = dh0 ? dh0 : fp(l.dh0);
    a.seqlen = seqlen;
    a.batch = batch;
    a.nheads = (int)nheads;
    a.dim = (int)dim;
    a.dstate = (int)dstate;
    a.euler = discretization == SSM_DISC_EULER ? 1 : 0;
    a.nchunks = l.nchunks;
    a.ngroups = l.ngroups;
    a.hbuf = fp(l.hbuf);
    a.gbuf = fp(l.gbuf);
    a.dd_part = fp(l.dd);
    a.db_part = fp(l.db);
    a.dc_part = fp(l.dc);
    a.da_part = fp(l.da);
    return hip_status(ssm::launch_ssd_bwd_mm(a, s));
  }
  int64_t chunk_len;
  int K;
  bwd_plan(seqlen, &chunk_len, &K);
  if (K > kMaxGridYZ) return SSM_ERR_UNSUPPORTED;
  const int io_bytes = io_dtype == SSM_DTYPE_BF16 ? 2 : 4;
  const SsdBwdLayout l = ssd_bwd_layout(batch, seqlen, dim, K, io_bytes);
  if (!workspace || workspace_bytes < l.total) return SSM_ERR_WORKSPACE;
  for (const void* p : ins)
    if (p && p == workspace) return SSM_ERR_INVALID_ARG;
  for (const void* o : outs)
    if (o && o == workspace) return SSM_ERR_INVALID_ARG;

  char* base = static_cast<char*>(workspace);
  void* delta_ch = base + l.delta_off;
  float* a_ch = reinterpret_cast<float*>(base + l.ach_off);
  float* da_ch = reinterpret_cast<float*>(base + l.dach_off);
  hipError_t e =
      ssm::launch_repeat_heads(dt, delta_ch, batch * seqlen, (int)nheads, (int)headdim, io_bytes, s);
  if (e == hipSuccess) e = ssm::launch_repeat_heads(A, a_ch, 1, (int)nheads, (int)headdim, 4, s);
  if (e != hipSuccess) return hip_status(e);

  ssm::BwdArgs a{};
  set_bwd_workspace(a, l.s.base, base, K);
  ssm::ScanArgs& f = a.f;
  f.x = x;
  f.delta = delta_ch;
  f.A = a_ch;
  f.B = B;
  f.C = C;
  f.Dskip = Dskip;
  f.z = z;
  f.h0 = h0;
  f.seqlen = seqlen;
  f.chunk_len = chunk_len;
  f.dim = (int)dim;
  f.batch = (int)batch;
  f.nchunks = K;
  f.a_per_channel = 1;
  f.euler = discretization == SSM_DISC_EULER ? 1 : 0;
  a.dy = dy;
  a.dh_last = dh_last;
  a.dx = dx;
  a.ddelta = base + l.ddch_off;
  a.dz = dz;
  a.dA = da_ch;
  a.dB = dB;
  a.dC = dC;
  a.dD = dD;
  a.dh0 = dh0;
  e = ssm::launch_scan_bwd_sliced(a, (int)dstate, io_dtype == SSM_DTYPE_BF16, base, l.s, s);
  // per-head gradients: the channels' fp32 ddelta sums and dA, summed per head
  if (e == hipSuccess)
    e = ssm::launch_sum_heads(reinterpret_cast<const float*>(base + l.s.accd_off), ddt,
                              batch * seqlen, (int)nheads, (int)headdim,
                              io_dtype == SSM_DTYPE_BF16 ? 1 : 0, s);
  if (e == hipSuccess)
    e = ssm::launch_sum_heads(da_ch, dA, 1, (int)nheads, (int)headdim, 0, s);
  return hip_status(e);
}

}  // extern "C"
