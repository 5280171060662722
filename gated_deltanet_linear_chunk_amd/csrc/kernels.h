// kernels.h -- launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

hipError_t launch_gate(const float* a, const float* b, const float* A_log, const float* dt_bias,
                       int64_t n_tokens, int H, float* g, float* beta, hipStream_t stream);

hipError_t launch_conv1d(const void* x, const void* w, const void* bias, int dt,
                         const int32_t* cu, int n_seqs, int B, int64_t T, int C, int width,
                         int apply_silu, int l2_channels, int head_dim, float l2_eps, int exact, void* y,
                         hipStream_t stream);

// Where the sequences of a chunk-rule launch come from and what they produce.
struct ChunkArgs {
  const void* q;  // [Ttot, Hqk, K] (may be null when no output is produced)
  const void* k;  // [Ttot, Hqk, K]
  const void* v;  // [Ttot, Hv, V]
  const float* g;     // [Ttot, Hv]
  const float* beta;  // [Ttot, Hv]
  const int32_t* cu;  // device offsets [n_seqs + 1] or null (then rows of row_len)
  int n_seqs;
  int64_t row_len;
  int64_t Ttot;
  int Hqk, Hv, K, V;
  // elements between consecutive tokens of q, k and v (dense: Hqk*K, Hqk*K, Hv*V)
  int64_t q_stride, k_stride, v_stride;
  float scale;
  int in_dt;  // 0 f32, 1 bf16
  // initial state: 0 zero, 1 load from s0 [n_seqs, Hv, K, V], 2 identity (augmented M columns)
  int s0_mode;
  const float* s0;
  void* o;  // [Ttot, Hv, V] or null
  int o_dt;
  // final state destination: element (seq, h, row i, col j) at
  // sf + seq * sf_seq_stride + h * sf_head_stride + i * sf_row_stride + j
  float* sf;
  int64_t sf_seq_stride, sf_head_stride, sf_row_stride;
  // bf16 path: per-(chunk slot, v-head) records of the state-independent chunk
  // quantities, chunk_slots(Ttot, n_seqs) * Hv * PREP_RECORD_BYTES bytes
  float* tbuf;
  // Optional maps of the bf16 scan (all null: block z runs sequence z, whose
  // start state follows s0_mode and whose final state goes to row z of sf).
  const int32_t* seq_order;  // [n_blocks_z]: sequence (of cu) that block z runs
  int n_blocks_z;            // grid z when seq_order is set
  const int32_t* s0_ref;     // [n_seqs]: >= 0 row of s0_seg, -1 zero, <= -2 row -2-r of s0
  const float* s0_seg;       // start states [*, Hv, K, V] picked by s0_ref
  const int32_t* sf_map;     // [n_seqs]: row of sf for the final state, -1 none
  // [n_seqs]: row of the records a sequence reads (the sample a segment cuts;
  // records are laid out by the offsets prep ran on), or null (its own index)
  const int32_t* rec_seq;
  int n_tiles;               // bf16 scan: column tiles per (sequence, v-head), set by its launcher
  // bf16 scan with V == 128: when z is set, o receives the gated RMS norm of
  // every output row, o * rsqrt(mean(o^2) + eps) * nw * silu(z), instead of o.
  const void* z;    // [Ttot, Hv, V] in z_dt (dense), or null
  int z_dt;         // 0 f32, 1 bf16
  const float* nw;  // [V] or null (ones)
  float eps;
  // fp32 kernel only: when cw is set, q, k and v point at the q | k | v
  // channel groups of one token-major buffer of raw conv inputs (k's group
  // starts Hqk*K channels after q's, v's 2*Hqk*K after), cw [channels,
  // conv_width] and cb [channels] (or null) are the depthwise conv's weights
  // and bias in in_dt, and the kernel forms q, k, v itself: conv over the
  // sequence's previous conv_width - 1 tokens (zero before its start), SiLU,
  // and q, k rows divided by sqrt(sum of squares + l2_eps) per head.
  const void* cw;
  const void* cb;
  int conv_width;
  float l2_eps;
  // bf16 MFMA path with the conv fused into the prep (chunk_prep_conv_kernel):
  // cx is the raw q | k | v channel input [tokens, 2*Hqk*K + Hv*V] (token
  // stride q_stride), cy the activations the prep stores in the same layout
  // (conv, SiLU, L2 norm of q and k rows; q, k, v point into it for the
  // scans), cw, cb, conv_width and l2_eps as above.
  const void* cx;
  void* cy;
  // Raw gate inputs (gdn_conv_chunk_fwd): when ga is set, the kernels form g
  // and beta themselves from ga, gb [Ttot, Hv] and gA_log, gdt_bias [Hv]
  // (gate_values) instead of reading g and beta.
  const float* ga;
  const float* gb;
  const float* gA_log;
  const float* gdt_bias;
};

// One record: T diag(beta) hi, lo (bf16, 10 tiles x 256 each), gamma[64] and
// dec[64] (fp32), then P hi, lo; a state-only scan reads just the part before P.
constexpr int PREP_REC_TB = 0;                        // 2 x 10 x 256 bf16
constexpr int PREP_REC_GAM = PREP_REC_TB + 2 * 10 * 256 * 2;
constexpr int PREP_REC_DEC = PREP_REC_GAM + 64 * 4;
constexpr int PREP_REC_P = PREP_REC_DEC + 64 * 4;     // 2 x 10 x 256 bf16
constexpr int PREP_RECORD_BYTES = PREP_REC_P + 2 * 10 * 256 * 2;

// Number of chunk slots a launch over Ttot tokens in n_seqs sequences uses.
int64_t chunk_slots(int64_t Ttot, int n_seqs);

hipError_t launch_chunk_f32(const ChunkArgs& a, hipStream_t stream);
// prep + scan; with prep = false the records in a.tbuf must already be there
hipError_t launch_chunk_bf16(const ChunkArgs& a, hipStream_t stream, bool prep = true);
// Pass 1 of the segment scan: M columns (v = 0, S0 = I) and b columns (S0 = 0),
// row z of M and b for block z.
hipError_t launch_segment_pass1(const ChunkArgs& a, float* M, float* b, hipStream_t stream,
                                bool prep = true);
// Pass 1 of a split run, one launch over a.n_blocks_z segments (those of
// a.seq_order, or the first ones; records already in a.tbuf): the first n_fwd run forward with
// outputs (start states by a.s0_ref, end states to rows a.sf_map of a.sf),
// the others form their maps as launch_segment_pass1 does, into row
// z - n_fwd of M and b.
hipError_t launch_split_pass1(const ChunkArgs& a, int n_fwd, float* M, float* b, hipStream_t stream);
// fp32 chains of affine maps.  chains[4 c .. 4 c + 3] = {n, p0, count, out0}:
// chain c starts from row n of s0 (zero when s0 is null or n < 0) and applies
// maps p0 .. p0 + count - 1 of (M, b) in order; with write_before, out row
// out0 + j receives the state before map j, else the state after it; final
// (when not null) row c receives the state after the last map.
// One chain of P maps from row 0 of s0, outputs as launch_compose_chains.
hipError_t launch_compose(const float* M, const float* b, const float* s0, int P, int Hv, int K,
                          int V, float* out, int write_before, float* final_state, hipStream_t stream);

// Stores n host values at dst (device) in stream order, carried inside kernel
// arguments kPlanArgInts at a time: the host buffer may be reused as soon as
// the call returns, and nothing waits for the stream.
constexpr int kPlanArgInts = 480;
struct PlanArg {
  int n;
  int32_t v[kPlanArgInts];
};
hipError_t launch_plan_store(const int32_t* ints, int64_t n, int32_t* dst, hipStream_t stream);
// The per-chunk records of a (with_p: also the output matrix P, which needs
// q).  When n_ints > 0 the same launch also stores ints[0, n_ints) at
// ints_dst, as launch_plan_store does.
hipError_t launch_chunk_prep(const ChunkArgs& a, int with_p, hipStream_t stream, const int32_t* ints = nullptr,
                             int64_t n_ints = 0, int32_t* ints_dst = nullptr);
hipError_t launch_compose_chains(const float* M, const float* b, const float* s0,
                                 const int32_t* chains, int n_chains, int Hv, int K, int V,
                                 float* out, int write_before, float* final_state,
                                 hipStream_t stream);

// One decode token per sequence on the fp32 state (see decode.hip).
struct DecodeArgs {
  const void* q;  // [N, Hqk, K] in in_dt
  const void* k;  // [N, Hqk, K]
  const void* v;  // [N, Hv, V]
  const float* g;     // [N, Hv]
  const float* beta;  // [N, Hv]
  float scale;
  float* state;                  // [n_state_rows, Hv, K, V], updated in place
  const int32_t* state_indices;  // [N] row of state per sequence (< 0: skip), or null (row n)
  int64_t n_state_rows;
  int N, Hqk, Hv, K, V;
  int in_dt, o_dt;  // 0 f32, 1 bf16
  void* o;          // [N, Hv, V]
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Output norm gated by z over rows of V values (see gated_norm.hip).
struct GatedNormArgs {
  const void* o;        // [rows, V] in o_dt
  const void* z;        // [rows, V] in z_dt
  const float* weight;  // [V] or null (ones)
  float eps;
  int64_t rows;
  int V;
  int o_dt, z_dt, y_dt;  // 0 f32, 1 bf16
  void* y;               // [rows, V] in y_dt
};
hipError_t launch_gated_norm(const GatedNormArgs& a, hipStream_t stream);

}  // namespace gdn
