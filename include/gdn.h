/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule forward library.
 *
 * The library computes the forward pass of a GatedDeltaNet linear-attention
 * layer's core: the gated delta rule recurrence (per head, a K x V state)
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,
 * evaluated chunk-parallel (64 tokens per chunk) on MFMA tiles, plus the steps
 * around it that the pages describe: the gates beta = sigmoid(b),
 * g = -exp(A_log) softplus(a + dt_bias); the causal depthwise conv1d + SiLU
 * over the concatenated q|k|v channels with packed samples that never see each
 * other (LlamaFactory PR "[v1] support GDN Ulysses cp", Design, decisions 5-7);
 * and the segment-wise affine state passing S_end = M S_start + b with a chain
 * of (M, b) reduced in fp32 (sglang fork PR "Qwen3.5 cp - #1", PR body and
 * Patches; prime-rl PR "feat: hybrid CP for Qwen3.5 MoE", Approach and
 * Communication-cost table), run here as a single-GPU segment-parallel scan;
 * the one-token recurrent step on cached states (sglang PR, the decode path
 * after the prefill); and the output RMS norm gated by z that follows the rule
 * (LlamaFactory PR, Design), on its own or applied by the chunk scan as it
 * writes o.  The state is stored K x V (prime-rl PR, Summary); the pages' V x K form
 * S (I - beta k k^T) is its transpose.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers to caller-owned, contiguous,
 *    row-major memory, 16-byte aligned.  The library allocates nothing and
 *    never frees or retains caller memory.  Its global state: the fixed
 *    device array of gdn_chunk_fwd_noalloc (present on every device the
 *    library's code is loaded on) and that array's per-device address; on the
 *    host, a cache of the last eight split plans (keyed by the offsets and
 *    sizes, behind a mutex), a per-device flag that the scan kernels' LDS
 *    limit is raised, and each device's compute-unit count.  Calls from several host threads are safe (calls of
 *    gdn_chunk_fwd_noalloc that overlap on one device race on its array).
 *  - Host pointers are named *_host and are read before the call returns.
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *    without waiting for it.  Results are valid once the stream reaches them.
 *  - Every call returns a gdn_status.  Argument errors are detected on the
 *    host before anything is enqueued, and then nothing is written.  A launch
 *    failure returns GDN_ERR_HIP.  No C++ exception crosses this boundary.
 *  - Packed samples: cu_seqlens (int32 [n_seqs + 1], device) holds sample
 *    offsets, cu[0] = 0, cu[n_seqs] = total tokens, non-decreasing.  It is
 *    only accepted with B == 1 (LlamaFactory PR, Design, decision 6).  Kernels
 *    clamp every offset into [0, T] so a malformed array cannot make them
 *    access memory out of bounds; pass the same array as cu_seqlens_host to
 *    have it validated (GDN_ERR_BAD_SEQLENS) before launch.  With
 *    GDN_VALIDATE=1 in the environment (read at every call), offsets given on
 *    the device alone are copied back and validated the same way; the call
 *    then waits for its stream, so this is for debugging, not for graph
 *    capture.  The same holds for the segment offsets of the segment entry
 *    points.
 *  - GQA: v-head h reads q/k head h / (H_v / H_qk) (contiguous groups).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  GDN_ERR_BAD_SHAPE = 2,    /* negative / inconsistent sizes */
  GDN_ERR_BAD_DTYPE = 3,    /* dtype code not accepted by this entry point */
  GDN_ERR_UNSUPPORTED = 4,  /* valid request for which the library has no kernel */
  GDN_ERR_BAD_SEQLENS = 5,  /* cu_seqlens / offsets malformed or with B > 1 */
  GDN_ERR_HIP = 6,          /* a HIP runtime call or kernel launch failed */
  GDN_ERR_SCRATCH_TOO_SMALL = 7 /* gdn_chunk_fwd_noalloc: input beyond its fixed array */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* How gdn_conv1d_fwd rounds its outputs (see there). */
typedef enum gdn_rounding { GDN_ROUND_FAST = 0, GDN_ROUND_EXACT = 1 } gdn_rounding;

/* Static text for a status code; never NULL. */
const char* gdn_status_string(int status);

/* ABI version of this header (incremented on any signature change). */
int gdn_abi_version(void);

/*
 * Gates (the pages' beta and g): for every token t and v-head h,
 *     beta[t, h] = 1 / (1 + exp(-b[t, h])),
 *     g[t, h]    = -exp(A_log[h]) * softplus(a[t, h] + dt_bias[h]),
 * softplus(x) = log(1 + exp(x)).  a, b, g, beta: fp32 [n_tokens, H];
 * A_log, dt_bias: fp32 [H].  g and beta are the gate inputs of
 * gdn_chunk_fwd.  n_tokens == 0 is a no-op.
 */
gdn_status gdn_gate_fwd(const float* a, const float* b, const float* A_log,
                        const float* dt_bias, int64_t n_tokens, int32_t H, float* g,
                        float* beta, hipStream_t stream);

/*
 * Causal depthwise conv1d over token-major channels, with optional SiLU and
 * optional per-head L2 normalisation (LlamaFactory PR, Design, decision 5:
 * the conv takes cu_seqlens so no sample sees another sample's tokens):
 *     z[t, c] = bias[c] + sum_{j=0}^{width-1} w[c, j] * x[t - width + 1 + j, c]
 * with x counted as 0 before the start of t's sample (or batch row);
 *     y = silu(z) = z / (1 + exp(-z)) when apply_silu, else z;
 * then, when l2norm_channels > 0, every group of head_dim consecutive
 * channels in [0, l2norm_channels) (the q and k heads) is divided by
 * sqrt(sum y^2 + l2_eps).  Accumulation is fp32; y is stored in `dt`.
 * rounding: GDN_ROUND_FAST stores the fp32 evaluation rounded once to `dt`
 * (round to nearest even; for bf16 within 2^-8 |y| + 1e-5 of the exact
 * value).  GDN_ROUND_EXACT (bf16 only; no effect on fp32 outputs) stores the
 * bf16 nearest to the exact value of every output, normalised or not: the
 * few fp32 results whose error bound straddles a rounding midpoint are
 * recomputed in fp64 (a normalised one with its whole head), which is slower.
 * Other values: GDN_ERR_BAD_SHAPE.
 *  x, y      [B, T, channels] in dt (f32 or bf16)
 *  w         [channels, width] in dt;  bias [channels] in dt or NULL
 *  cu_seqlens device int32 [n_seqs + 1] or NULL (then B rows of T tokens)
 *  width in [1, 4]; channels % 8 == 0; l2norm_channels % head_dim == 0;
 *  head_dim a power of two in [8, 512] when l2norm_channels > 0.
 */
gdn_status gdn_conv1d_fwd(const void* x, const void* w, const void* bias, gdn_dtype dt,
                          const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                          int32_t n_seqs, int32_t B, int64_t T, int32_t channels,
                          int32_t width, int32_t apply_silu, int32_t l2norm_channels,
                          int32_t head_dim, float l2_eps, gdn_rounding rounding, void* y,
                          hipStream_t stream);

/*
 * Chunked gated delta rule forward (chunk size 64).  For every sequence n
 * (a cu_seqlens sample, or a batch row) and v-head h, starting from
 * initial_state[n, h] (zero when NULL), the recurrence above runs over the
 * sequence's tokens; o[t, h] = scale * S_t^T q_t, and final_state[n, h]
 * receives the state after the last token (the sglang PR hands this state to
 * the decode path).  The chunk grid is anchored at each sequence start; a
 * zero-length sequence copies initial_state to final_state.
 *  q, k   [B, T, H_qk, K] in in_dt        v   [B, T, H_v, V] in in_dt
 *  g,beta fp32 [B, T, H_v]                o   [B, T, H_v, V] in o_dt
 *  initial_state, final_state fp32 [N, H_v, K, V], N = n_seqs (packed) or B;
 *  either may be NULL.
 *  *_token_stride: elements between consecutive tokens of q, k, v (0 = dense:
 *  H_qk*K, H_qk*K, H_v*V).  A larger stride reads q, k, v straight out of a
 *  wider token-major buffer, e.g. the conv1d output [T, q|k|v channels];
 *  strides must be multiples of 8, at least the dense size and below 2^24
 *  elements (GDN_ERR_BAD_SHAPE otherwise).  The B
 *  batch rows are then B*T tokens at that stride.
 * Kernels: in_dt = BF16 with K = 128 and V % 128 == 0 runs bf16 MFMA tiles
 * with fp32 accumulation, an fp32 state, and split-bf16 operands where fp32
 * intermediates meet the matrix cores; every other supported shape (K in
 * {32, 64, 128}, V % 32 == 0, in_dt F32 or BF16) runs an fp32 vector-ALU
 * kernel on the inputs as given (GDN_ERR_UNSUPPORTED otherwise).
 * o_dt is F32 or BF16 (round to nearest even).
 * workspace: device memory of at least gdn_chunk_fwd_workspace_bytes(...)
 * bytes (0 for the vector-ALU shapes; NULL allowed then).  The MFMA path stores there,
 * per 64-token chunk and v-head, the state-independent matrices of the UT
 * transform (products of T = (I + A)^{-1}, the masked Q K^T, the decays),
 * which a parallel pass computes before the serial chunk scan; contents on
 * entry do not matter.  Concurrent calls need separate workspaces.
 */
size_t gdn_chunk_fwd_workspace_bytes(gdn_dtype in_dt, int64_t total_tokens, int32_t n_seqs,
                                     int32_t H_v, int32_t K, int32_t V);

gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                         int64_t q_token_stride, int64_t k_token_stride, int64_t v_token_stride,
                         const float* g, const float* beta, float scale,
                         const float* initial_state, const int32_t* cu_seqlens,
                         const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t B, int64_t T,
                         int32_t H_qk, int32_t H_v, int32_t K, int32_t V, void* o,
                         gdn_dtype o_dt, float* final_state, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as gdn_chunk_fwd without the workspace:
 * the per-chunk records of the BF16 path live in a fixed device array of
 * GDN_NOALLOC_SCRATCH_BYTES bytes built into the library (one per device,
 * held until the process ends).  They take 20992 * H_v * (ceil(total/64) + N)
 * bytes (total tokens, N sequences), which must fit
 * (GDN_ERR_SCRATCH_TOO_SMALL otherwise; e.g. 8192 tokens in up to 71
 * sequences at H_v = 32).  Packed runs are never segment-split here, so the
 * call makes no host-to-device copy; it enqueues kernels only, and allocates
 * and frees nothing.  Every call on one device shares that device's array:
 * calls that overlap in time on one device (different streams, or threads)
 * race and give wrong results; calls in one stream are ordered and safe.
 * `stream` must belong to the current device (GDN_ERR_UNSUPPORTED otherwise).
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                                 int64_t q_token_stride, int64_t k_token_stride,
                                 int64_t v_token_stride, const float* g, const float* beta,
                                 float scale, const float* initial_state,
                                 const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                 int32_t n_seqs, int32_t B, int64_t T, int32_t H_qk, int32_t H_v,
                                 int32_t K, int32_t V, void* o, gdn_dtype o_dt,
                                 float* final_state, hipStream_t stream);

/*
 * gdn_chunk_fwd followed by the gated output norm of gdn_gated_rmsnorm_fwd,
 * "chunk_gated_delta_rule + norm" with the z component (LlamaFactory PR
 * "[v1] support GDN Ulysses cp", Design; the norm's form is the per-head RMS
 * norm gated by SiLU(z) stated at gdn_gated_rmsnorm_fwd):
 *     o[t, h] = n / sqrt(mean(n^2) + eps) * norm_weight * z[t, h] sigmoid(z[t, h]),
 *     n = scale * S_t^T q_t  (the output gdn_chunk_fwd would store).
 * Arguments as in gdn_chunk_fwd, plus z [B, T, H_v, V] in z_dt (dense, o's
 * layout), norm_weight fp32 [V] or NULL (ones), eps >= 0 (GDN_ERR_BAD_SHAPE
 * otherwise).  On the MFMA path with V = 128 the scan applies the norm to
 * its fp32 output rows as it writes them, so n never reaches memory; other
 * shapes run gdn_chunk_fwd into o and then the norm in place over o (V in
 * {32, 64, 128, 256, 512}, GDN_ERR_UNSUPPORTED otherwise), with n rounded
 * to o_dt in between.  Workspace as for gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_gated_norm(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                                    int64_t q_token_stride, int64_t k_token_stride,
                                    int64_t v_token_stride, const float* g, const float* beta,
                                    float scale, const float* initial_state,
                                    const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                    int32_t n_seqs, int32_t B, int64_t T, int32_t H_qk, int32_t H_v,
                                    int32_t K, int32_t V, const void* z, gdn_dtype z_dt,
                                    const float* norm_weight, float eps, void* o, gdn_dtype o_dt,
                                    float* final_state, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * The short convolution, SiLU and q/k L2 norm of gdn_conv1d_fwd fused into
 * the chunk rule's load stage.  The pages run the depthwise conv over the
 * concatenated q | k | v channels and hand its output to the chunk rule on
 * the same token-major layout (LlamaFactory PR "[v1] support GDN Ulysses
 * cp", Design: one conv over the joined q, k, v channels feeds the chunk rule); here
 * the chunk kernels form each 64-token chunk's q, k, v rows from the raw
 * channels themselves:
 *     a[t, c] = silu(bias[c] + sum_{j<width} w[c, j] x[t - width + 1 + j, c])
 * with x zero before the first token of t's sequence, and every q and k
 * head row divided by sqrt(sum of squares + l2_eps) -- the activations of
 * gdn_conv1d_fwd with l2norm_channels = 2 H_qk K, head_dim = K -- then run
 * the rule of gdn_chunk_fwd on them.
 *  x     [B, T, C] in in_dt, dense, C = 2 H_qk K + H_v V channels in the order
 *        q heads | k heads | v heads
 *  w     [C, width] in in_dt, width in [1, 4];  bias [C] in in_dt or NULL
 *  l2_eps > 0 (GDN_ERR_BAD_SHAPE otherwise)
 *  a, b  fp32 [B, T, H_v] gate inputs, A_log, dt_bias fp32 [H_v]: the call
 *        forms g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b)
 *        itself, with the arithmetic of gdn_gate_fwd
 *  scale, initial_state, cu_seqlens, cu_seqlens_host, n_seqs, B, T, H_qk,
 *  H_v, K, V, o, o_dt, final_state: as gdn_chunk_fwd.
 * Kernels: bf16 inputs with K = 128, V % 128 == 0 and H_v / H_qk <= 4 run
 * the MFMA path with the conv in its chunk prep: the prep stores the
 * activations as bf16 into the workspace, computed exactly as
 * gdn_conv1d_fwd with GDN_ROUND_FAST computes them, so o and final_state
 * equal the unfused steps (gdn_gate_fwd and gdn_conv1d_fwd, then
 * gdn_chunk_fwd on their outputs) bit for bit; packed calls with host offsets are split as gdn_chunk_fwd
 * splits them.  Every other shape (K in {32, 64, 128}, V % 32 == 0;
 * GDN_ERR_UNSUPPORTED otherwise) runs the fp32 vector-ALU kernel, which keeps
 * the activations in fp32, never writes them and needs no workspace: each of
 * its workgroups forms the q, k rows of its head and the v columns of its
 * slice.
 *  workspace: device memory of at least gdn_conv_chunk_fwd_workspace_bytes
 *  bytes (0 for shapes of the vector-ALU kernel, where it may be NULL); its
 *  contents on entry do not matter.  GDN_ERR_NULL_POINTER when a workspace is
 *  needed and missing, GDN_ERR_BAD_SHAPE when it is too small.
 */
size_t gdn_conv_chunk_fwd_workspace_bytes(gdn_dtype in_dt, int64_t total_tokens, int32_t n_seqs,
                                          int32_t H_qk, int32_t H_v, int32_t K, int32_t V);
gdn_status gdn_conv_chunk_fwd(const void* x, const void* w, const void* bias, gdn_dtype in_dt,
                              int32_t width, float l2_eps, const float* a, const float* b,
                              const float* A_log, const float* dt_bias, float scale, const float* initial_state, const int32_t* cu_seqlens,
                              const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t B, int64_t T,
                              int32_t H_qk, int32_t H_v, int32_t K, int32_t V, void* o,
                              gdn_dtype o_dt, float* final_state, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * Segment state scan: one long sequence cut into P contiguous segments
 * [seg_offsets[i], seg_offsets[i+1]) of the token arrays (the sglang PR's
 * per-rank segments, here on one GPU).  Pass 1 computes, for every segment
 * and v-head, the affine map of the segment, S_end = M S_start + b
 * (M: K x K, the product of the segment's per-token transitions; b: the state
 * reached from a zero start), by running the chunked rule on the augmented
 * state [M | b] started at [I | 0].  The maps are then composed in fp32,
 * S_start,0 = initial_state (zero when NULL), S_start,i+1 = M_i S_start,i + b_i.
 *  k [T, H_qk, K], v [T, H_v, V] in in_dt with K = 128 and V % 32 == 0
 *  (GDN_ERR_UNSUPPORTED otherwise): bf16 with V % 128 == 0 runs the MFMA
 *  kernels, fp32 inputs and other V the fp32 vector-ALU kernel (pass 1 as
 *  two runs of the rule, M's columns from the identity with zero values and
 *  b's from zero); the composition is fp32 MFMA for both;
 *  token strides as in gdn_chunk_fwd (0 = dense);
 *  g, beta fp32 [T, H_v]; seg_offsets device int32 [P + 1] (host mirror
 *  seg_offsets_host optional, validated when given);
 *  initial_state fp32 [H_v, K, V] or NULL;
 *  M fp32 [P, H_v, K, K] and b fp32 [P, H_v, K, V] (outputs, required);
 *  seg_initial_states fp32 [P, H_v, K, V] (output, required);
 *  final_state fp32 [H_v, K, V] or NULL (the state after the last segment).
 * Running gdn_chunk_fwd with cu_seqlens = seg_offsets (seg_offsets[0] = 0,
 * seg_offsets[P] = T) and initial_state = seg_initial_states is pass 2: it
 * yields every output of the unsegmented run.
 * workspace: at least gdn_segment_state_scan_workspace_bytes(...) bytes
 * (the per-chunk UT-transform matrices of pass 1) on the MFMA shapes; not
 * used, and NULL allowed, on the vector-ALU shapes.
 */
size_t gdn_segment_state_scan_workspace_bytes(int64_t T, int32_t P, int32_t H_v, int32_t K,
                                              int32_t V);

gdn_status gdn_segment_state_scan(const void* k, const void* v, gdn_dtype in_dt,
                                  int64_t k_token_stride, int64_t v_token_stride,
                                  const float* g, const float* beta,
                                  const int32_t* seg_offsets, const int32_t* seg_offsets_host,
                                  int32_t P, const float* initial_state, int64_t T,
                                  int32_t H_qk, int32_t H_v, int32_t K, int32_t V, float* M,
                                  float* b, float* seg_initial_states, float* final_state,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Segment-parallel forward of one long sequence: the segments' affine maps
 * (pass 1), their fp32 composition into start states, then the forward over
 * the segments from those starts (pass 2).  On the MFMA kernels pass 1 runs
 * segment 0 forward beside the maps of segments 1 .. P-2 and the chain
 * starts from segment 0's end state, so P = 2 with the cut at a multiple of
 * 64 tokens gives the unsegmented result bit for bit; on the vector-ALU
 * kernel pass 1 forms the maps of segments 0 .. P-2 as
 * gdn_segment_state_scan does.  Same q/k/v/g/beta/o layouts as
 * gdn_chunk_fwd with B = 1; seg_offsets as above with seg_offsets[0] = 0 and
 * seg_offsets[P] = T.  final_state fp32 [H_v, K, V] or NULL.  Shapes and
 * kernels as gdn_segment_state_scan.
 * workspace: device memory of at least gdn_segmented_workspace_bytes(...)
 * bytes, used for M, b, the composed starts, the start and final-state maps
 * and (MFMA shapes) the per-chunk matrices; its contents on entry do not
 * matter.
 */
size_t gdn_segmented_workspace_bytes(int64_t T, int32_t P, int32_t H_v, int32_t K, int32_t V);

gdn_status gdn_chunk_fwd_segmented(const void* q, const void* k, const void* v,
                                   gdn_dtype in_dt, int64_t q_token_stride,
                                   int64_t k_token_stride, int64_t v_token_stride,
                                   const float* g, const float* beta,
                                   float scale, const float* initial_state,
                                   const int32_t* seg_offsets, const int32_t* seg_offsets_host,
                                   int32_t P, int64_t T, int32_t H_qk, int32_t H_v, int32_t K,
                                   int32_t V, void* o, gdn_dtype o_dt, float* final_state,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Recurrent decode step: one new token for each of N sequences, on states
 * kept by the caller (the sglang fork PR "Qwen3.5 cp - #1" hands the final
 * state of the prefill to the standard decode path; PR body).  For sequence
 * n and v-head h, with S = state[r, h] (K x V, fp32) and r = state_indices[n]
 * (r = n when state_indices is NULL), the recurrence above advances one token
 * in place:  S <- e^g S; u = beta (v - S^T k); S <- S + k u^T;
 * o[n, h] = scale * S^T q.  A row r < 0 or >= n_state_rows skips sequence n:
 * its o is zero and no state is touched (padding slots of a serving batch).
 * Two sequences must not name the same row.
 *  q, k  [N, H_qk, K] in in_dt     v [N, H_v, V] in in_dt
 *  g,beta fp32 [N, H_v]            o [N, H_v, V] in o_dt
 *  state fp32 [n_state_rows, H_v, K, V]; state_indices int32 [N] (device) or NULL.
 * K in {32, 64, 128}, V % 32 == 0, N <= 65535; all arithmetic in fp32.
 */
gdn_status gdn_decode_step(const void* q, const void* k, const void* v, gdn_dtype in_dt,
                           const float* g, const float* beta, float scale, float* state,
                           const int32_t* state_indices, int64_t n_state_rows, int32_t N,
                           int32_t H_qk, int32_t H_v, int32_t K, int32_t V, void* o,
                           gdn_dtype o_dt, hipStream_t stream);

/*
 * Output norm gated by z, the step after the chunk rule ("chunk_gated_delta_rule
 * + norm" with the z component: LlamaFactory PR "[v1] support GDN Ulysses cp",
 * Design; the pages give no formula, this is a per-head RMS norm gated by
 * SiLU(z)).  For every row r (one token of one v-head) of V values:
 *   y[r] = o[r] / sqrt(mean(o[r]^2) + eps) * weight * z[r] sigmoid(z[r]).
 *  o [rows, V] in o_dt, z [rows, V] in z_dt, weight fp32 [V] or NULL (ones),
 *  y [rows, V] in y_dt (may be o when both dtypes and shapes agree: each row is
 *  read before it is written by the same threads).
 * V in {32, 64, 128, 256, 512}; eps >= 0; fp32 arithmetic.
 */
gdn_status gdn_gated_rmsnorm_fwd(const void* o, gdn_dtype o_dt, const void* z, gdn_dtype z_dt,
                                 const float* weight, float eps, int64_t rows, int32_t V, void* y,
                                 gdn_dtype y_dt, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
