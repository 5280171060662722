// api.cpp -- the extern "C" entry points declared in include/gdn.h.
//
// Host side only: argument validation (before anything is enqueued), choice of
// kernel, and the launches.  Nothing here allocates device memory or
// synchronises the host with the stream; the only global state is the fixed
// device array of gdn_chunk_fwd_noalloc and its per-device addresses.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "kernels.h"
#include "split_plan.h"

namespace {

constexpr int kAbiVersion = 3;
constexpr int kMaxGrid = 65535;

gdn_status hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

bool valid_dtype(int dt) { return dt == GDN_F32 || dt == GDN_BF16; }

// Host mirror of packed offsets: cu[0] == first, non-decreasing, cu[n] == last.
bool offsets_ok(const int32_t* cu, int32_t n, int64_t first_max, int64_t last, bool exact_ends) {
  if (!cu || n < 1) return false;
  if (cu[0] < 0 || cu[0] > first_max) return false;
  if (exact_ends && cu[0] != 0) return false;
  for (int32_t i = 0; i < n; ++i)
    if (cu[i + 1] < cu[i]) return false;
  if (cu[n] > last) return false;
  if (exact_ends && cu[n] != last) return false;
  return true;
}

// GDN_VALIDATE=1 in the environment (read at every call): offsets passed on
// the device alone are copied back and checked like a host mirror, and the
// call waits for `stream` up to that copy.  A debugging aid: it blocks the
// host and cannot be captured into a graph.
bool validate_device_offsets() {
  const char* e = std::getenv("GDN_VALIDATE");
  return e && e[0] == '1' && e[1] == 0;
}

// Offsets check of an entry point: the host mirror when given, else (with
// GDN_VALIDATE=1) a host copy of the device array; n >= 1.
gdn_status check_offsets(const int32_t* dev, const int32_t* host, int32_t n, int64_t first_max, int64_t last,
                         bool exact_ends, hipStream_t stream) {
  if (host) return offsets_ok(host, n, first_max, last, exact_ends) ? GDN_OK : GDN_ERR_BAD_SEQLENS;
  if (!dev || !validate_device_offsets()) return GDN_OK;
  std::vector<int32_t> copy((size_t)n + 1);
  if (hipMemcpyAsync(copy.data(), dev, sizeof(int32_t) * copy.size(), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return GDN_ERR_HIP;
  return offsets_ok(copy.data(), n, first_max, last, exact_ends) ? GDN_OK : GDN_ERR_BAD_SEQLENS;
}

// Token stride: 0 selects the dense value; otherwise a multiple of 8, >= dense.
// Below 2^24 elements, so that the kernels form a lane's offset inside a
// 64-token chunk with one 24-bit multiply.
bool stride_ok(int64_t* stride, int64_t dense) {
  if (*stride == 0) *stride = dense;
  return *stride >= dense && *stride % 8 == 0 && *stride < (int64_t(1) << 24);
}

// The bf16 MFMA kernels (with their per-chunk records) take K = 128 and V a
// multiple of 128; every other supported shape (K in {32, 64, 128}, V a
// multiple of 32, either input dtype) runs the fp32 vector-ALU kernel.
bool mfma_path(int in_dt, int32_t K, int32_t V) { return in_dt == GDN_BF16 && K == 128 && V > 0 && V % 128 == 0; }

// Which chunk kernel serves (in_dt, K, V); GDN_OK when one does.
gdn_status chunk_supported(int in_dt, int32_t K, int32_t V) {
  if (mfma_path(in_dt, K, V)) return GDN_OK;
  if (K == 32 || K == 64 || K == 128) return (V > 0 && V % 32 == 0) ? GDN_OK : GDN_ERR_UNSUPPORTED;
  return GDN_ERR_UNSUPPORTED;
}

size_t tbuf_bytes(int64_t Ttot, int32_t n_seqs, int32_t H_v) {
  return (size_t)gdn::PREP_RECORD_BYTES * (size_t)gdn::chunk_slots(Ttot, n_seqs) * (size_t)H_v;
}

// Compute units of the current device, queried once per device.
int device_cus() {
  static std::atomic<int> known[64];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && (n = known[dev].load(std::memory_order_relaxed)) > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
  if (dev >= 0 && dev < 64) known[dev].store(n, std::memory_order_relaxed);
  return n;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of a split run: records of the N samples (laid out as for the
// unsplit run), M and b of the pass-1 segments, start states of the later
// segments, the plan's index arrays.
size_t split_workspace_bytes(int64_t total, int N, int n_seg, int n_prefix, int32_t H_v, int32_t K, int32_t V) {
  const size_t st = (size_t)H_v * K * V * sizeof(float);
  return align256(tbuf_bytes(total, N, H_v)) + align256((size_t)n_prefix * H_v * K * K * sizeof(float)) +
         2 * align256((size_t)n_prefix * st) +
         align256(sizeof(int32_t) * (size_t)gdn::split_plan_ints_max(n_seg, n_prefix));
}

// Segment shapes: bf16 with K = 128 and V % 128 == 0 on the MFMA kernels;
// K = 128 with V % 32 == 0 otherwise (either dtype) on the fp32 vector-ALU
// kernel, whose maps the same fp32 composition chains.
gdn_status segment_supported(int in_dt, int32_t K, int32_t V) {
  if (mfma_path(in_dt, K, V)) return GDN_OK;
  return (K == 128 && V > 0 && V % 32 == 0) ? GDN_OK : GDN_ERR_UNSUPPORTED;
}

// Pass 1 on the vector-ALU kernel: the augmented state [M | b] of each of the
// a.n_seqs segments as two runs of the rule, M's K columns from the identity
// with zero values, b's V columns from zero with the values.
hipError_t segment_pass1_f32(const gdn::ChunkArgs& a, float* M, float* b, hipStream_t stream) {
  gdn::ChunkArgs m = a;
  m.q = nullptr;
  m.v = nullptr;
  m.o = nullptr;
  m.V = a.K;
  m.s0_mode = 2;
  m.s0 = nullptr;
  m.s0_ref = nullptr;
  m.sf_map = nullptr;
  m.sf = M;
  m.sf_seq_stride = (int64_t)a.Hv * a.K * a.K;
  m.sf_head_stride = (int64_t)a.K * a.K;
  m.sf_row_stride = a.K;
  hipError_t e = gdn::launch_chunk_f32(m, stream);
  if (e != hipSuccess) return e;
  gdn::ChunkArgs c = a;
  c.q = nullptr;
  c.o = nullptr;
  c.s0_mode = 0;
  c.s0 = nullptr;
  c.s0_ref = nullptr;
  c.sf_map = nullptr;
  c.sf = b;
  c.sf_seq_stride = (int64_t)a.Hv * a.K * a.V;
  c.sf_head_stride = (int64_t)a.K * a.V;
  c.sf_row_stride = a.V;
  return gdn::launch_chunk_f32(c, stream);
}

}  // namespace

extern "C" {

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "negative or inconsistent sizes";
    case GDN_ERR_BAD_DTYPE: return "dtype not accepted by this entry point";
    case GDN_ERR_UNSUPPORTED: return "no kernel for this combination of sizes and dtype";
    case GDN_ERR_BAD_SEQLENS: return "malformed cu_seqlens / segment offsets, or offsets with B > 1";
    case GDN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case GDN_ERR_SCRATCH_TOO_SMALL:
      return "the request needs more than the fixed scratch array of gdn_chunk_fwd_noalloc holds";
    default: return "unknown status";
  }
}

int gdn_abi_version(void) { return kAbiVersion; }

gdn_status gdn_gate_fwd(const float* a, const float* b, const float* A_log, const float* dt_bias,
                        int64_t n_tokens, int32_t H, float* g, float* beta, hipStream_t stream) {
  if (n_tokens < 0 || H <= 0) return GDN_ERR_BAD_SHAPE;
  if (n_tokens == 0) return GDN_OK;
  if (!a || !b || !A_log || !dt_bias || !g || !beta) return GDN_ERR_NULL_POINTER;
  return hip_status(gdn::launch_gate(a, b, A_log, dt_bias, n_tokens, H, g, beta, stream));
}

gdn_status gdn_conv1d_fwd(const void* x, const void* w, const void* bias, gdn_dtype dt,
                          const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                          int32_t n_seqs, int32_t B, int64_t T, int32_t channels,
                          int32_t width, int32_t apply_silu, int32_t l2norm_channels,
                          int32_t head_dim, float l2_eps, gdn_rounding rounding, void* y,
                          hipStream_t stream) {
  if (!valid_dtype(dt)) return GDN_ERR_BAD_DTYPE;
  if (rounding != GDN_ROUND_FAST && rounding != GDN_ROUND_EXACT) return GDN_ERR_BAD_SHAPE;
  if (B < 1 || T < 0 || channels <= 0 || channels % 8 != 0) return GDN_ERR_BAD_SHAPE;
  if (width < 1 || width > 4) return GDN_ERR_UNSUPPORTED;
  if (l2norm_channels < 0 || l2norm_channels > channels) return GDN_ERR_BAD_SHAPE;
  if (l2norm_channels > 0) {
    if (head_dim < 8 || head_dim > 512 || (head_dim & (head_dim - 1)) != 0) return GDN_ERR_UNSUPPORTED;
    if (l2norm_channels % head_dim != 0) return GDN_ERR_BAD_SHAPE;
  }
  if (cu_seqlens) {
    if (B != 1 || n_seqs < 1) return GDN_ERR_BAD_SEQLENS;
    const gdn_status cs = check_offsets(cu_seqlens, cu_seqlens_host, n_seqs, 0, T, true, stream);
    if (cs != GDN_OK) return cs;
  }
  const int64_t total = (int64_t)B * T;
  if (total == 0) return GDN_OK;
  if (!x || !w || !y) return GDN_ERR_NULL_POINTER;
  if ((total + 31) / 32 > kMaxGrid) return GDN_ERR_UNSUPPORTED;
  return hip_status(gdn::launch_conv1d(x, w, bias, dt, cu_seqlens, n_seqs, B, T, channels, width,
                                       apply_silu, l2norm_channels, head_dim, l2_eps,
                                       rounding == GDN_ROUND_EXACT ? 1 : 0, y, stream));
}

size_t gdn_chunk_fwd_workspace_bytes(gdn_dtype in_dt, int64_t total_tokens, int32_t n_seqs,
                                     int32_t H_v, int32_t K, int32_t V) {
  if (!mfma_path(in_dt, K, V) || total_tokens < 0 || n_seqs < 0 || H_v < 1) return 0;
  const size_t plain = tbuf_bytes(total_tokens, n_seqs, H_v);
  const int pmax = gdn::max_prefix_segments(H_v, V, device_cus());
  if (pmax == 0 || n_seqs < 1) return plain;
  return std::max(plain, split_workspace_bytes(total_tokens, n_seqs, n_seqs + pmax, pmax, H_v, K, V));
}

// The gated output norm that the bf16 scan applies as it writes o (null: none).
struct FusedNorm {
  const void* z;
  int z_dt;
  const float* weight;
  float eps;
};

// The short convolution in front of the MFMA path (gdn_conv_chunk_fwd): raw
// channels x, taps, bias, width and eps, y, the buffer the prep stores the
// activations to (q, k, v of the run point into it), and the raw gate inputs
// the prep forms g and beta from.
struct ConvIn {
  const void* x;
  const void* w;
  const void* bias;
  int width;
  float eps;
  void* y;
  const float *ga, *gb, *gA_log, *gdt_bias;
};

// Source of the records' memory for callers without a workspace: called once
// the arguments are validated, with the sizes of the bf16 run; sets the
// workspace, or returns why it cannot.  Runs that use it are never split.
typedef gdn_status (*FixedWorkspace)(hipStream_t stream, int64_t total, int32_t n_seqs, int32_t H_v,
                                     void** workspace, size_t* workspace_bytes);

static gdn_status chunk_fwd_run(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                         int64_t q_token_stride, int64_t k_token_stride, int64_t v_token_stride,
                         const float* g, const float* beta, float scale,
                         const float* initial_state, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t B, int64_t T,
                         int32_t H_qk, int32_t H_v, int32_t K, int32_t V, void* o,
                         gdn_dtype o_dt, float* final_state, void* workspace,
                         size_t workspace_bytes, const FusedNorm* norm, hipStream_t stream,
                         FixedWorkspace fixed_ws = nullptr, const ConvIn* conv = nullptr) {
  if (!valid_dtype(in_dt) || !valid_dtype(o_dt)) return GDN_ERR_BAD_DTYPE;
  if (B < 1 || T < 0 || H_qk < 1 || H_v < 1 || K < 1 || V < 1) return GDN_ERR_BAD_SHAPE;
  if (H_v % H_qk != 0) return GDN_ERR_BAD_SHAPE;
  if (!stride_ok(&q_token_stride, (int64_t)H_qk * K) || !stride_ok(&k_token_stride, (int64_t)H_qk * K) ||
      !stride_ok(&v_token_stride, (int64_t)H_v * V))
    return GDN_ERR_BAD_SHAPE;
  if (cu_seqlens) {
    if (B != 1 || n_seqs < 1) return GDN_ERR_BAD_SEQLENS;
    const gdn_status cs = check_offsets(cu_seqlens, cu_seqlens_host, n_seqs, 0, T, true, stream);
    if (cs != GDN_OK) return cs;
  }
  const gdn_status sup = chunk_supported(in_dt, K, V);
  if (sup != GDN_OK) return sup;
  const int32_t N = cu_seqlens ? n_seqs : B;
  if (N > kMaxGrid || H_v > kMaxGrid) return GDN_ERR_UNSUPPORTED;
  const int64_t total = cu_seqlens ? T : (int64_t)B * T;
  if (total == 0 && !final_state) return GDN_OK;
  const bool raw_gates = conv && conv->ga;
  if (total > 0 && (!q || !k || !v || (!raw_gates && (!g || !beta)) || !o)) return GDN_ERR_NULL_POINTER;
  const bool mfma = mfma_path(in_dt, K, V);
  if (mfma) {
    if (fixed_ws) {
      const gdn_status st = fixed_ws(stream, total, N, H_v, &workspace, &workspace_bytes);
      if (st != GDN_OK) return st;
    }
    if (!workspace) return GDN_ERR_NULL_POINTER;
    if (workspace_bytes < tbuf_bytes(total, N, H_v)) return GDN_ERR_BAD_SHAPE;
  }
  gdn::ChunkArgs a{};
  a.tbuf = static_cast<float*>(workspace);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu = cu_seqlens;
  a.n_seqs = N;
  a.row_len = T;
  a.Ttot = total;
  a.Hqk = H_qk;
  a.Hv = H_v;
  a.K = K;
  a.V = V;
  a.q_stride = q_token_stride;
  a.k_stride = k_token_stride;
  a.v_stride = v_token_stride;
  a.scale = scale;
  a.in_dt = in_dt;
  a.s0_mode = initial_state ? 1 : 0;
  a.s0 = initial_state;
  a.o = o;
  a.o_dt = o_dt;
  a.sf = final_state;
  a.sf_seq_stride = (int64_t)H_v * K * V;
  a.sf_head_stride = (int64_t)K * V;
  a.sf_row_stride = V;
  if (norm) {
    if (total > 0 && !norm->z) return GDN_ERR_NULL_POINTER;
    a.z = norm->z;
    a.z_dt = norm->z_dt;
    a.nw = norm->weight;
    a.eps = norm->eps;
  }
  if (!mfma) return hip_status(gdn::launch_chunk_f32(a, stream));
  if (conv) {
    a.cx = conv->x;
    a.cy = conv->y;
    a.cw = conv->w;
    a.cb = conv->bias;
    a.conv_width = conv->width;
    a.l2_eps = conv->eps;
    a.ga = conv->ga;
    a.gb = conv->gb;
    a.gA_log = conv->gA_log;
    a.gdt_bias = conv->gdt_bias;
  }
  // A split plan (cached for repeated offsets) comes first, so that the prep
  // launch on the samples also stores its index arrays.
  gdn::SplitPlan plan;
  bool split = false;
  if (!fixed_ws && cu_seqlens && cu_seqlens_host && total > 0)
    split = gdn::plan_split(cu_seqlens_host, N, H_v, V, initial_state != nullptr, device_cus(), plan) &&
            workspace_bytes >= split_workspace_bytes(total, N, plan.n_seg, plan.n_prefix, H_v, K, V);
  if (!split) {
    const hipError_t e = gdn::launch_chunk_prep(a, (o && q) ? 1 : 0, stream);
    if (e != hipSuccess) return GDN_ERR_HIP;
    return hip_status(gdn::launch_chunk_bf16(a, stream, false));
  }
  // ---- segment-split run (see plan_split) ----------------------------------------
  unsigned char* w = static_cast<unsigned char*>(workspace);
  const size_t st = (size_t)H_v * K * V;
  w += align256(tbuf_bytes(total, N, H_v));
  float* M = reinterpret_cast<float*>(w);
  w += align256((size_t)plan.n_prefix * H_v * K * K * sizeof(float));
  float* bmap = reinterpret_cast<float*>(w);
  w += align256((size_t)plan.n_prefix * st * sizeof(float));
  float* starts = reinterpret_cast<float*>(w);
  w += align256((size_t)plan.n_prefix * st * sizeof(float));
  int32_t* ints = reinterpret_cast<int32_t*>(w);
  hipError_t e = gdn::launch_chunk_prep(a, (o && q) ? 1 : 0, stream, plan.ints.data(), (int64_t)plan.ints.size(),
                                        ints);
  if (e != hipSuccess) return GDN_ERR_HIP;
  a.cu = ints;
  a.n_seqs = plan.n_seg;
  a.rec_seq = ints + plan.off_sample();
  // pass 1: the first segment of every split sample forward, its end state to
  // the start row of the sample's second segment; the middle segments' maps
  gdn::ChunkArgs p1 = a;
  p1.seq_order = ints + plan.off_pre();
  p1.n_blocks_z = plan.n_prefix;
  p1.s0_ref = ints + plan.off_s0ref();
  p1.s0_seg = starts;
  p1.sf = starts;
  p1.sf_map = ints + plan.off_s0ref() + 1;  // segment i ends where segment i + 1 starts
  e = gdn::launch_split_pass1(p1, plan.n_fwd, M, bmap, stream);
  if (e != hipSuccess) return GDN_ERR_HIP;
  // chains from each second segment's start through the maps
  e = gdn::launch_compose_chains(M, bmap, starts, ints + plan.off_chains(), plan.n_chain, H_v, K, V, starts, 0,
                                 nullptr, stream);
  if (e != hipSuccess) return GDN_ERR_HIP;
  gdn::ChunkArgs p2 = a;
  p2.seq_order = ints + plan.off_order();
  p2.n_blocks_z = plan.n_seg - plan.n_fwd;
  p2.s0_ref = ints + plan.off_s0ref();
  p2.s0_seg = starts;
  p2.sf_map = ints + plan.off_sfmap();
  return hip_status(gdn::launch_chunk_bf16(p2, stream, false));
}

gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                         int64_t q_token_stride, int64_t k_token_stride, int64_t v_token_stride,
                         const float* g, const float* beta, float scale,
                         const float* initial_state, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t B, int64_t T,
                         int32_t H_qk, int32_t H_v, int32_t K, int32_t V, void* o,
                         gdn_dtype o_dt, float* final_state, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return chunk_fwd_run(q, k, v, in_dt, q_token_stride, k_token_stride, v_token_stride, g, beta, scale,
                       initial_state, cu_seqlens, cu_seqlens_host, n_seqs, B, T, H_qk, H_v, K, V, o, o_dt,
                       final_state, workspace, workspace_bytes, nullptr, stream);
}

}  // extern "C"

namespace {

// The records of gdn_chunk_fwd_noalloc.  Every GPU the library runs on holds
// its own copy of this array until the process ends; host code uses the
// per-device address that hipGetSymbolAddress returns, never the name.
constexpr size_t kScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// Address of `scratch` on the device of `stream` (which must be current),
// looked up once per device.
gdn_status scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return GDN_ERR_HIP;
    if (sdev != dev) return GDN_ERR_UNSUPPORTED;
  }
  if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

// FixedWorkspace over `scratch`: the size limit first, then the address.  The
// records are written in full before they are read, so nothing is cleared.
gdn_status scratch_workspace(hipStream_t stream, int64_t total, int32_t n_seqs, int32_t H_v,
                             void** workspace, size_t* workspace_bytes) {
  if (gdn::chunk_slots(total, n_seqs) > (int64_t)(kScratchBytes / ((size_t)gdn::PREP_RECORD_BYTES * (size_t)H_v)))
    return GDN_ERR_SCRATCH_TOO_SMALL;
  const gdn_status st = scratch_address(stream, workspace);
  if (st != GDN_OK) return st;
  *workspace_bytes = kScratchBytes;
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                                 int64_t q_token_stride, int64_t k_token_stride,
                                 int64_t v_token_stride, const float* g, const float* beta,
                                 float scale, const float* initial_state,
                                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                 int32_t n_seqs, int32_t B, int64_t T, int32_t H_qk, int32_t H_v,
                                 int32_t K, int32_t V, void* o, gdn_dtype o_dt,
                                 float* final_state, hipStream_t stream) {
  return chunk_fwd_run(q, k, v, in_dt, q_token_stride, k_token_stride, v_token_stride, g, beta, scale,
                       initial_state, cu_seqlens, cu_seqlens_host, n_seqs, B, T, H_qk, H_v, K, V, o, o_dt,
                       final_state, nullptr, 0, nullptr, stream, scratch_workspace);
}

gdn_status gdn_chunk_fwd_gated_norm(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                                    int64_t q_token_stride, int64_t k_token_stride,
                                    int64_t v_token_stride, const float* g, const float* beta,
                                    float scale, const float* initial_state,
                                    const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                    int32_t n_seqs, int32_t B, int64_t T, int32_t H_qk, int32_t H_v,
                                    int32_t K, int32_t V, const void* z, gdn_dtype z_dt,
                                    const float* norm_weight, float eps, void* o, gdn_dtype o_dt,
                                    float* final_state, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  if (!valid_dtype(in_dt) || !valid_dtype(o_dt) || !valid_dtype(z_dt)) return GDN_ERR_BAD_DTYPE;
  if (!(eps >= 0.f)) return GDN_ERR_BAD_SHAPE;
  if (mfma_path(in_dt, K, V) && V == 128) {
    const FusedNorm norm{z, z_dt == GDN_BF16 ? 1 : 0, norm_weight, eps};
    return chunk_fwd_run(q, k, v, in_dt, q_token_stride, k_token_stride, v_token_stride, g, beta, scale,
                         initial_state, cu_seqlens, cu_seqlens_host, n_seqs, B, T, H_qk, H_v, K, V, o,
                         o_dt, final_state, workspace, workspace_bytes, &norm, stream);
  }
  // other shapes: the chunk forward, then the norm kernel over o in place
  if (V != 32 && V != 64 && V != 128 && V != 256 && V != 512) return GDN_ERR_UNSUPPORTED;
  const int64_t total = cu_seqlens ? T : (int64_t)B * T;
  if (total > 0 && !z) return GDN_ERR_NULL_POINTER;
  // the norm kernel's own limit, checked before anything is enqueued
  const int64_t rpb = 256 / (V / 8);
  if (total > 0 && (total * H_v + rpb - 1) / rpb > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  const gdn_status st = chunk_fwd_run(q, k, v, in_dt, q_token_stride, k_token_stride, v_token_stride, g,
                                      beta, scale, initial_state, cu_seqlens, cu_seqlens_host, n_seqs, B, T,
                                      H_qk, H_v, K, V, o, o_dt, final_state, workspace, workspace_bytes,
                                      nullptr, stream);
  if (st != GDN_OK || total <= 0) return st;
  return gdn_gated_rmsnorm_fwd(o, o_dt, z, z_dt, norm_weight, eps, total * H_v, V, o, o_dt, stream);
}

// The MFMA path with the conv in its prep: bf16, the MFMA head sizes, and at
// most four v-heads per q/k head (one workgroup of the prep holds them all).
static bool conv_chunk_mfma(gdn_dtype in_dt, int32_t H_qk, int32_t H_v, int32_t K, int32_t V) {
  return in_dt == GDN_BF16 && mfma_path(in_dt, K, V) && H_qk > 0 && H_v % H_qk == 0 && H_v / H_qk <= 4;
}

size_t gdn_conv_chunk_fwd_workspace_bytes(gdn_dtype in_dt, int64_t total_tokens, int32_t n_seqs,
                                          int32_t H_qk, int32_t H_v, int32_t K, int32_t V) {
  if (!conv_chunk_mfma(in_dt, H_qk, H_v, K, V) || total_tokens < 0 || n_seqs < 0) return 0;
  const int64_t C = 2 * (int64_t)H_qk * K + (int64_t)H_v * V;
  return align256((size_t)total_tokens * (size_t)C * 2) +
         gdn_chunk_fwd_workspace_bytes(in_dt, total_tokens, n_seqs, H_v, K, V);
}

gdn_status gdn_conv_chunk_fwd(const void* x, const void* w, const void* bias, gdn_dtype in_dt,
                              int32_t width, float l2_eps, const float* ga, const float* gb,
                              const float* A_log, const float* dt_bias, float scale, const float* initial_state, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t B, int64_t T,
                              int32_t H_qk, int32_t H_v, int32_t K, int32_t V, void* o,
                              gdn_dtype o_dt, float* final_state, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(in_dt) || !valid_dtype(o_dt)) return GDN_ERR_BAD_DTYPE;
  if (B < 1 || T < 0 || H_qk < 1 || H_v < 1 || K < 1 || V < 1) return GDN_ERR_BAD_SHAPE;
  if (H_v % H_qk != 0 || !(l2_eps > 0.f)) return GDN_ERR_BAD_SHAPE;
  if (width < 1 || width > 4) return GDN_ERR_UNSUPPORTED;
  if ((K != 32 && K != 64 && K != 128) || V % 32 != 0) return GDN_ERR_UNSUPPORTED;
  const int64_t C = 2 * (int64_t)H_qk * K + (int64_t)H_v * V;
  int64_t stride = C;
  if (!stride_ok(&stride, C)) return GDN_ERR_BAD_SHAPE;
  if (cu_seqlens) {
    if (B != 1 || n_seqs < 1) return GDN_ERR_BAD_SEQLENS;
    const gdn_status cs = check_offsets(cu_seqlens, cu_seqlens_host, n_seqs, 0, T, true, stream);
    if (cs != GDN_OK) return cs;
  }
  const int32_t N = cu_seqlens ? n_seqs : B;
  if (N > kMaxGrid || H_v > kMaxGrid) return GDN_ERR_UNSUPPORTED;
  const int64_t total = cu_seqlens ? T : (int64_t)B * T;
  if (total == 0 && !final_state) return GDN_OK;
  if (total > 0 && (!x || !w || !ga || !gb || !A_log || !dt_bias || !o)) return GDN_ERR_NULL_POINTER;
  const size_t es = in_dt == GDN_BF16 ? 2 : 4;
  if (conv_chunk_mfma(in_dt, H_qk, H_v, K, V)) {
    // the activations take the front of the workspace, the chunk rule the rest
    if (!workspace) return GDN_ERR_NULL_POINTER;
    if (workspace_bytes < gdn_conv_chunk_fwd_workspace_bytes(in_dt, total, N, H_qk, H_v, K, V))
      return GDN_ERR_BAD_SHAPE;
    const size_t ybytes = align256((size_t)total * (size_t)C * es);
    unsigned char* y = static_cast<unsigned char*>(workspace);
    const ConvIn conv{x, w, bias, width, l2_eps, y, ga, gb, A_log, dt_bias};
    return chunk_fwd_run(y, y + es * (size_t)H_qk * K, y + es * 2 * (size_t)H_qk * K, in_dt, C, C, C, nullptr, nullptr,
                         scale, initial_state, cu_seqlens, cu_seqlens_host, n_seqs, B, T, H_qk, H_v, K, V, o,
                         o_dt, final_state, y + ybytes, workspace_bytes - ybytes, nullptr, stream, nullptr, &conv);
  }
  const unsigned char* xb = static_cast<const unsigned char*>(x);
  gdn::ChunkArgs a{};
  a.q = xb;
  a.k = xb ? xb + es * (size_t)H_qk * K : nullptr;
  a.v = xb ? xb + es * 2 * (size_t)H_qk * K : nullptr;
  a.ga = ga;
  a.gb = gb;
  a.gA_log = A_log;
  a.gdt_bias = dt_bias;
  a.cu = cu_seqlens;
  a.n_seqs = N;
  a.row_len = T;
  a.Ttot = total;
  a.Hqk = H_qk;
  a.Hv = H_v;
  a.K = K;
  a.V = V;
  a.q_stride = a.k_stride = a.v_stride = stride;
  a.scale = scale;
  a.in_dt = in_dt;
  a.s0_mode = initial_state ? 1 : 0;
  a.s0 = initial_state;
  a.o = o;
  a.o_dt = o_dt;
  a.sf = final_state;
  a.sf_seq_stride = (int64_t)H_v * K * V;
  a.sf_head_stride = (int64_t)K * V;
  a.sf_row_stride = V;
  a.cw = w;
  a.cb = bias;
  a.conv_width = width;
  a.l2_eps = l2_eps;
  // A zero-token call only copies the start states; the plain kernel does that.
  if (total == 0) a.cw = nullptr;
  return hip_status(gdn::launch_chunk_f32(a, stream));
}

size_t gdn_segment_state_scan_workspace_bytes(int64_t T, int32_t P, int32_t H_v, int32_t K,
                                              int32_t V) {
  (void)K;
  (void)V;
  if (T < 0 || P < 1 || H_v < 1) return 0;
  return tbuf_bytes(T, P, H_v);
}

gdn_status gdn_segment_state_scan(const void* k, const void* v, gdn_dtype in_dt,
                                  int64_t k_token_stride, int64_t v_token_stride,
                                  const float* g, const float* beta,
                                  const int32_t* seg_offsets, const int32_t* seg_offsets_host,
                                  int32_t P, const float* initial_state, int64_t T,
                                  int32_t H_qk, int32_t H_v, int32_t K, int32_t V, float* M,
                                  float* b, float* seg_initial_states, float* final_state,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(in_dt)) return GDN_ERR_BAD_DTYPE;
  if (P < 1 || T < 0 || H_qk < 1 || H_v < 1 || H_v % H_qk != 0) return GDN_ERR_BAD_SHAPE;
  const gdn_status sup = segment_supported(in_dt, K, V);
  if (sup != GDN_OK) return sup;
  const bool mfma = mfma_path(in_dt, K, V);
  if (P > kMaxGrid || H_v > kMaxGrid) return GDN_ERR_UNSUPPORTED;
  if (!stride_ok(&k_token_stride, (int64_t)H_qk * K) || !stride_ok(&v_token_stride, (int64_t)H_v * V))
    return GDN_ERR_BAD_SHAPE;
  if (!seg_offsets) return GDN_ERR_NULL_POINTER;
  const gdn_status cs = check_offsets(seg_offsets, seg_offsets_host, P, T, T, false, stream);
  if (cs != GDN_OK) return cs;
  if (!k || !v || !g || !beta || !M || !b || !seg_initial_states) return GDN_ERR_NULL_POINTER;
  if (mfma && !workspace) return GDN_ERR_NULL_POINTER;
  if (mfma && workspace_bytes < tbuf_bytes(T, P, H_v)) return GDN_ERR_BAD_SHAPE;
  gdn::ChunkArgs a{};
  a.tbuf = static_cast<float*>(workspace);
  a.q = nullptr;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu = seg_offsets;
  a.n_seqs = P;
  a.row_len = T;
  a.Ttot = T;
  a.Hqk = H_qk;
  a.Hv = H_v;
  a.K = K;
  a.V = V;
  a.q_stride = k_token_stride;
  a.k_stride = k_token_stride;
  a.v_stride = v_token_stride;
  a.scale = 1.f;
  a.in_dt = in_dt;
  a.s0_mode = 0;
  a.o_dt = GDN_F32;
  hipError_t e = mfma ? gdn::launch_segment_pass1(a, M, b, stream) : segment_pass1_f32(a, M, b, stream);
  if (e != hipSuccess) return GDN_ERR_HIP;
  e = gdn::launch_compose(M, b, initial_state, P, H_v, K, V, seg_initial_states, 1, final_state, stream);
  return hip_status(e);
}

}  // extern "C"

namespace {

// Workspace of gdn_chunk_fwd_segmented: records of the P segments, M, b and
// start states of the P - 1 segments that precede another, and the start /
// final-state maps of pass 2.
struct SegmentedLayout {
  size_t rec, M, b, starts, ints, total;
};

SegmentedLayout segmented_layout(int64_t T, int32_t P, int32_t H_v, int32_t K, int32_t V) {
  SegmentedLayout l;
  const size_t pre = (size_t)(P - 1) * H_v * K;
  l.rec = 0;
  l.M = l.rec + align256(tbuf_bytes(T, P, H_v));
  l.b = l.M + align256(pre * K * sizeof(float));
  l.starts = l.b + align256(pre * V * sizeof(float));
  l.ints = l.starts + align256(pre * V * sizeof(float));
  l.total = l.ints + align256((3 * (size_t)P + 3) * sizeof(int32_t));
  return l;
}

}  // namespace

extern "C" {

size_t gdn_segmented_workspace_bytes(int64_t T, int32_t P, int32_t H_v, int32_t K, int32_t V) {
  if (T < 0 || P < 1 || H_v < 1 || K < 1 || V < 1) return 0;
  return segmented_layout(T, P, H_v, K, V).total;
}

// Prep once for all P segments (the records with P serve both passes).  On
// the MFMA kernels pass 1 runs segment 0 forward (its end state is the start
// of segment 1) beside the maps of segments 1 .. P-2, one fp32 chain carries
// segment 1's start through those maps, and pass 2 runs segments 1 .. P-1
// from the chained starts; on the vector-ALU kernel pass 1 forms the maps of
// segments 0 .. P-2, the chain starts from initial_state, and pass 2 runs all
// P segments.  Pass 2 writes the final state.
gdn_status gdn_chunk_fwd_segmented(const void* q, const void* k, const void* v,
                                   gdn_dtype in_dt, int64_t q_token_stride,
                                   int64_t k_token_stride, int64_t v_token_stride,
                                   const float* g, const float* beta,
                                   float scale, const float* initial_state,
                                   const int32_t* seg_offsets, const int32_t* seg_offsets_host,
                                   int32_t P, int64_t T, int32_t H_qk, int32_t H_v, int32_t K,
                                   int32_t V, void* o, gdn_dtype o_dt, float* final_state,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // every check before anything is enqueued
  if (!valid_dtype(in_dt) || !valid_dtype(o_dt)) return GDN_ERR_BAD_DTYPE;
  if (P < 1 || T < 0 || H_qk < 1 || H_v < 1 || H_v % H_qk != 0) return GDN_ERR_BAD_SHAPE;
  const gdn_status sup = segment_supported(in_dt, K, V);
  if (sup != GDN_OK) return sup;
  const bool mfma = mfma_path(in_dt, K, V);
  if (P > kMaxGrid || H_v > kMaxGrid) return GDN_ERR_UNSUPPORTED;
  if (!stride_ok(&q_token_stride, (int64_t)H_qk * K) || !stride_ok(&k_token_stride, (int64_t)H_qk * K) ||
      !stride_ok(&v_token_stride, (int64_t)H_v * V))
    return GDN_ERR_BAD_SHAPE;
  const gdn_status cs = check_offsets(seg_offsets, seg_offsets_host, P, 0, T, true, stream);
  if (cs != GDN_OK) return cs;
  if (!seg_offsets || !workspace) return GDN_ERR_NULL_POINTER;
  if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL_POINTER;
  const SegmentedLayout l = segmented_layout(T, P, H_v, K, V);
  if (workspace_bytes < l.total) return GDN_ERR_BAD_SHAPE;
  if (T == 0 && !final_state) return GDN_OK;

  unsigned char* w = static_cast<unsigned char*>(workspace);
  float* M = reinterpret_cast<float*>(w + l.M);
  float* bmap = reinterpret_cast<float*>(w + l.b);
  float* starts = reinterpret_cast<float*>(w + l.starts);
  int32_t* ints = reinterpret_cast<int32_t*>(w + l.ints);
  // s0_ref [P]: segment 0 starts from row 0 of initial_state (zero when
  // NULL), segment i > 0 from start row i - 1; sf_map [P]: the last segment's
  // state is the final state; then the MFMA path's chain (from start row 0
  // through maps 0 .. P-3 to start rows 1 .. P-2) and its pass-2 order
  // (segments 1 .. P-1)
  const bool mixed = mfma && P > 1 && T > 0;
  std::vector<int32_t> maps(2 * (size_t)P, -1);
  maps[0] = -2;
  for (int32_t i = 1; i < P; ++i) maps[i] = i - 1;
  maps[(size_t)P + P - 1] = 0;
  if (mixed) {
    const int32_t chain[4] = {0, 0, P - 2, 1};
    maps.insert(maps.end(), chain, chain + 4);
    for (int32_t i = 1; i < P; ++i) maps.push_back(i);
  }
  gdn::ChunkArgs a{};
  a.tbuf = reinterpret_cast<float*>(w + l.rec);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.cu = seg_offsets;
  a.n_seqs = P;
  a.row_len = T;
  a.Ttot = T;
  a.Hqk = H_qk;
  a.Hv = H_v;
  a.K = K;
  a.V = V;
  a.q_stride = q_token_stride;
  a.k_stride = k_token_stride;
  a.v_stride = v_token_stride;
  a.scale = scale;
  a.in_dt = in_dt;
  a.s0_mode = 0;
  a.s0 = initial_state;
  a.o = o;
  a.o_dt = o_dt;
  a.sf = final_state;
  a.sf_seq_stride = (int64_t)H_v * K * V;
  a.sf_head_stride = (int64_t)K * V;
  a.sf_row_stride = V;
  // the maps go to the device with the prep launch (or a store of their own)
  hipError_t e = mfma ? gdn::launch_chunk_prep(a, T > 0 ? 1 : 0, stream, maps.data(), (int64_t)maps.size(), ints)
                      : gdn::launch_plan_store(maps.data(), (int64_t)maps.size(), ints, stream);
  if (e != hipSuccess) return GDN_ERR_HIP;
  if (mixed) {
    gdn::ChunkArgs p1 = a;
    p1.n_blocks_z = P - 1;  // segment 0 forward, segments 1 .. P-2 maps
    p1.s0_ref = ints;
    p1.s0_seg = starts;
    p1.sf = starts;
    p1.sf_map = ints + 1;  // segment 0 ends where segment 1 starts
    e = gdn::launch_split_pass1(p1, 1, M, bmap, stream);
    if (e != hipSuccess) return GDN_ERR_HIP;
    e = gdn::launch_compose_chains(M, bmap, starts, ints + 2 * P, P > 2 ? 1 : 0, H_v, K, V, starts, 0, nullptr,
                                   stream);
    if (e != hipSuccess) return GDN_ERR_HIP;
  } else if (P > 1) {
    gdn::ChunkArgs p1 = a;
    p1.n_seqs = P - 1;  // segments 0 .. P-2: the same chunk slots as in the P-segment records
    e = mfma ? gdn::launch_segment_pass1(p1, M, bmap, stream, false) : segment_pass1_f32(p1, M, bmap, stream);
    if (e != hipSuccess) return GDN_ERR_HIP;
    e = gdn::launch_compose(M, bmap, initial_state, P - 1, H_v, K, V, starts, 0, nullptr, stream);
    if (e != hipSuccess) return GDN_ERR_HIP;
  }
  gdn::ChunkArgs p2 = a;
  p2.s0_ref = ints;
  p2.s0_seg = starts;
  p2.sf_map = ints + P;
  if (mixed) {
    p2.seq_order = ints + 2 * P + 4;
    p2.n_blocks_z = P - 1;
  }
  if (T == 0) {
    p2.q = nullptr;  // no tokens: the state-only scan copies initial_state to final_state
    p2.o = nullptr;
  }
  return hip_status(mfma ? gdn::launch_chunk_bf16(p2, stream, false) : gdn::launch_chunk_f32(p2, stream));
}


gdn_status gdn_decode_step(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                           const float* g, const float* beta, float scale, float* state,
                           const int32_t* state_indices, int64_t n_state_rows, int32_t N,
                           int32_t H_qk, int32_t H_v, int32_t K, int32_t V, void* o,
                           gdn_dtype o_dt, hipStream_t stream) {
  if (!valid_dtype(in_dt) || !valid_dtype(o_dt)) return GDN_ERR_BAD_DTYPE;
  if (N < 0 || H_qk < 1 || H_v < 1 || K < 1 || V < 1 || n_state_rows < 0) return GDN_ERR_BAD_SHAPE;
  if (H_v % H_qk != 0) return GDN_ERR_BAD_SHAPE;
  if (!state_indices && n_state_rows < N) return GDN_ERR_BAD_SHAPE;
  if ((K != 32 && K != 64 && K != 128) || V % 32 != 0 || N > 65535) return GDN_ERR_UNSUPPORTED;
  if (N == 0) return GDN_OK;
  if (!q || !k || !v || !g || !beta || !state || !o) return GDN_ERR_NULL_POINTER;
  gdn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.scale = scale;
  a.state = state;
  a.state_indices = state_indices;
  a.n_state_rows = n_state_rows;
  a.N = N;
  a.Hqk = H_qk;
  a.Hv = H_v;
  a.K = K;
  a.V = V;
  a.in_dt = in_dt == GDN_BF16 ? 1 : 0;
  a.o_dt = o_dt == GDN_BF16 ? 1 : 0;
  a.o = o;
  return hip_status(gdn::launch_decode(a, stream));
}

gdn_status gdn_gated_rmsnorm_fwd(const void* o, gdn_dtype o_dt, const void* z, gdn_dtype z_dt,
                                 const float* weight, float eps, int64_t rows, int32_t V, void* y,
                                 gdn_dtype y_dt, hipStream_t stream) {
  if (!valid_dtype(o_dt) || !valid_dtype(z_dt) || !valid_dtype(y_dt)) return GDN_ERR_BAD_DTYPE;
  if (rows < 0 || V < 1 || !(eps >= 0.f)) return GDN_ERR_BAD_SHAPE;
  if (V != 32 && V != 64 && V != 128 && V != 256 && V != 512) return GDN_ERR_UNSUPPORTED;
  const int rpb = 256 / (V / 8);
  if ((rows + rpb - 1) / rpb > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  if (rows == 0) return GDN_OK;
  if (!o || !z || !y) return GDN_ERR_NULL_POINTER;
  gdn::GatedNormArgs a;
  a.o = o;
  a.z = z;
  a.weight = weight;
  a.eps = eps;
  a.rows = rows;
  a.V = V;
  a.o_dt = o_dt == GDN_BF16 ? 1 : 0;
  a.z_dt = z_dt == GDN_BF16 ? 1 : 0;
  a.y_dt = y_dt == GDN_BF16 ? 1 : 0;
  a.y = y;
  return hip_status(gdn::launch_gated_norm(a, stream));
}

}  // extern "C"
