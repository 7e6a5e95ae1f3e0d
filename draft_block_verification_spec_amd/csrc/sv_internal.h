// Internal declarations shared by the HIP translation units of libspecverify.
// Not part of the public ABI (see include/spec_verify.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

// ---------------------------------------------------------------- vector types
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Per-row partial statistics of a logit row over a subset of its columns:
// b1 = max z, b2 = second largest z, i1 = lowest column index attaining b1,
// s = sum over the subset of exp((z - b1) * invT).  Empty: b1 = b2 = -inf, s = 0.
struct alignas(16) StatPart {
  float b1, b2, s;
  int i1;
};

enum Epilogue : int {
  EPI_LOGITS = 0,  // fp32 logits (optional) + per-row StatPart partials
  EPI_SWIGLU = 1,  // a = bf16(silu(g) * u), g/u from paired weight rows
  EPI_RESID = 2,   // y = bf16(resid + acc)
  EPI_RAW = 3,     // fp32 split-K partial, no epilogue
};

// Arguments of the GEMM kernels: out[m, n] = sum_k X[m, k] * W[n, k].
// X rows m < m1 come from x1 (row stride ldx1), rows m1 <= m < M from x2.
struct GemmArgs {
  const uint16_t *x1;
  const uint16_t *x2;
  long ldx1, ldx2;
  int m1;
  int M;             // rows (upper bound when M_dev is given)
  const int *M_dev;  // optional device-side row count (scheduled mode)
  // With M_dev: the launch does its work only when m_lo < *M_dev and, if m_hi > 0,
  // *M_dev <= m_hi (a plan for few rows and one for many, both launched, one working)
  int m_lo, m_hi;
  // EPI_LOGITS: when set, the launch that does the work writes nslots_plan (the statistics
  // slots per row of the whole product, all launches of its plan) here
  int32_t *nslots_out;
  int nslots_plan;
  int N;             // output columns (for SWIGLU: columns of a)
  int K;             // reduction length, multiple of 64
  const uint16_t *w;   // [N, K] (SWIGLU: gate rows)
  const uint16_t *w2;  // SWIGLU: up rows [N, K]
  // EPI_LOGITS
  float *logits;  // may be null
  long ldl;
  StatPart *parts;
  int nslots;
  float invT;
  int want_s;  // compute the sum-exp part of the statistics
  // EPI_SWIGLU / EPI_RESID
  uint16_t *out;
  long ldo;
  const uint16_t *resid;
  long ldr;
  // EPI_RAW (split-K partials [splits][M][Ncols])
  float *partial;
  // zeroed by thread 0 of block 0 before anything else (device status, arrival counter)
  int32_t *status_reset;
  int32_t *counter_reset;  // counter_reset[0 .. counter_reset_n) are zeroed (n >= 1 when set)
  int counter_reset_n;
  int buf_cols;  // set by the streaming launcher: columns of the per-workgroup output buffer
  int n_off;     // EPI_LOGITS: column index of output column 0 (argmax indices of a later launch)
  // FP8 (E4M3) weights: w / w2 hold one code per element and every output row n is
  // multiplied by wscale[n] (w) / wscale2[n] (w2); weight-streaming kernel only
  int wfp8;
  const float *wscale;
  const float *wscale2;
};

// Sampling job: draw v from w_v = max(0, exp(z1_v*invT - lse1) - [z2 ? exp(z2_v*invT - lse2) : 0])
// by inverse CDF with coin u; if the weights sum to zero, fall back to exp(z1_v*invT - lse1).
struct SampleJob {
  const float *z1;
  const float *z2;  // may be null
  float lse1, lse2;
  float u;
  int out_index;  // index into the int32 output array
};

// Number of compute units of the current device (cached).
int num_cus();

// ---------------------------------------------------------------- launchers
hipError_t launch_gemm_stream(const GemmArgs &a, int epi, int grid, hipStream_t st);
int stream_grid(const GemmArgs &a, int epi);
bool stream_ok(int M, int epi);

// Tile shape of the LDS-tiled GEMM: BM x BN outputs per workgroup, k-slices of BK
// values, NS slices in the LDS pipeline.
struct TileShape {
  int bm, bn, bk, ns;
};
// Shape chosen for an M x N x K product with epilogue epi (K must be a multiple of 64).
TileShape tiled_shape(int M, int N, int K, int epi);
// Workgroups of a shape resident per CU (LDS and waves per SIMD).
int tiled_per_cu(const TileShape &sh);
hipError_t launch_gemm_tiled(const GemmArgs &a, int epi, const TileShape &sh, int splits, hipStream_t st);
// Statistics slots per row of an EPI_LOGITS launch over N columns (one per column tile
// and wave column).
int tiled_slots(int N, const TileShape &sh);
hipError_t launch_splitk_reduce(const GemmArgs &a, int epi, int splits, int bn, hipStream_t st);

// End-of-call bookkeeping (tau and counters), run by the last block of the last kernel.
struct FinalizeArgs {
  const int32_t *acc;   // accepted lengths [B]; null = skip
  const int32_t *vlen;  // verified drafts per request [B] (scheduled), else null (K each)
  int B, K;
  float *tau;
  int64_t *counters;
};

struct AcceptArgs {
  int B, K, V;  // K = Kmax in scheduled mode
  float invT;
  const StatPart *parts_t;  // target-row partials [rows][nslots_t]
  int nslots_t;
  const int32_t *nslots_t_dev;  // when set, nslots_t as written by the LM-head launch that ran
  const StatPart *parts_d;  // draft-row partials [B*K][nslots_d]
  int nslots_d;
  const float *logits_t;  // target logits (packed rows in scheduled mode), row stride V
  const float *logits_d;  // draft logits, row stride V
  const int32_t *draft;   // [B, K]
  const float *u;         // [B, K+1]
  const int32_t *verify_len;  // scheduled: k_b, else null
  const int32_t *row_off;     // scheduled: packed target row base per request, else null
  int32_t *accepted_len;
  int32_t *emitted;
  SampleJob *jobs;  // one per request (sample / scheduled)
  int32_t *dev_status;
  float *diag;  // may be null
  int32_t *job_cnt;   // sampling arrival counters [B] (zeroed here)
  int32_t *done_cnt;  // call-wide arrival counter (zeroed here in sampled modes; greedy: zeroed earlier)
  FinalizeArgs fin;   // greedy: bookkeeping by the last block
};
hipError_t launch_accept_sample(const AcceptArgs &a, hipStream_t st);
hipError_t launch_accept_greedy(const AcceptArgs &a, hipStream_t st);

int sample_chunks(int V);
// Small batches (B*(K+1) <= 32): acceptance decided in every chunk block, then the
// weights and the draw of the accepted candidate only.  sums [B*C*2] (chunk sums of
// max(0, p-q) and p), req [3*B] (first rejection A as int bits, then the two normalisers).
hipError_t launch_tail_small(const AcceptArgs &a, float *sums, float *req, const FinalizeArgs &fin,
                             hipStream_t st);
hipError_t launch_sample(const SampleJob *jobs, int njobs, int V, float invT, float *chunk_sums,
                         int32_t *out, int32_t *job_cnt, int32_t *done_cnt, const FinalizeArgs &fin,
                         hipStream_t st);

hipError_t launch_init(int32_t *zero_i32, size_t n_i32, int32_t *dev_status, hipStream_t st);

struct ScheduleArgs {
  int B, Kmax, V;
  float invT, threshold;
  int budget;
  const StatPart *parts_d;
  int nslots_d;
  int32_t *verify_len;  // [B]
  int32_t *row_off;     // [B+1]
  int32_t *row_map;     // [budget] packed row -> b*(Kmax+1)+j
  int32_t *m_total;     // [1]
  float *conf;          // [B*Kmax]
  int32_t *dev_status;
  int32_t *verify_len_out;  // optional copy for the caller
  int32_t *status_reset;    // zeroed first when non-null
  float *diag;              // optional per-row records; draft rows start at row diag_row0
  long diag_row0;
};
hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t st);
hipError_t launch_gather_rows(const uint16_t *src, uint16_t *dst, const int32_t *row_map,
                              const int32_t *m_total, int max_rows, int d, hipStream_t st);
hipError_t launch_scatter_logits(const float *packed, float *dst, const int32_t *row_map,
                                 const int32_t *m_total, int max_rows, int V, hipStream_t st);
hipError_t launch_scatter_hidden(const uint16_t *packed, uint16_t *dst, const int32_t *row_map,
                                 const int32_t *m_total, int max_rows, int d, hipStream_t st);
hipError_t launch_propose_finish(const StatPart *parts, int nslots, int rows, float invT, float T,
                                 const float *logits, int V, const float *coins, SampleJob *jobs,
                                 int32_t *draft_out, float *conf_out, int32_t *dev_status,
                                 int32_t *job_cnt, hipStream_t st);

// Tree verification tail (see spec_verify_tree): one block per request.
struct TreeArgs {
  int B, K, V;
  float invT;   // 1 when greedy
  int greedy;
  const StatPart *parts_t;  // [B*(K+1)][nslots_t]
  int nslots_t;
  const StatPart *parts_d;  // [B*K][nslots_d] (sampled)
  int nslots_d;
  const float *logits_t;  // [B*(K+1), V] (sampled)
  const float *logits_d;  // [B*K, V] (sampled)
  const int32_t *tokens;  // [B, K]
  const int32_t *parent;  // [B, K]
  const float *u;         // [B, K+1] (sampled)
  int32_t *accepted_len, *emitted, *path;
  int32_t *dev_status;
  float *diag;
  int32_t *done_cnt;
  FinalizeArgs fin;
  // sampled trees over several blocks per request (zeroed counters, see launch_tree)
  float *chunk_sums;  // [B][tree_chunks(V)]
  float *partials;    // [B][2][TREE_MAX_BLOCKS]
  int32_t *meet;      // [B] block arrival counters, zero on entry
  int spin_limit;     // bounded wait of a block for the others (iterations)
};
constexpr int TREE_MAX_BLOCKS = 16;
int tree_chunks(int V);
// Sampled trees spread each residual pass over up to TREE_MAX_BLOCKS co-resident blocks
// per request when chunk_sums is set and the device allows a cooperative launch;
// otherwise one block per request.
hipError_t launch_tree(const TreeArgs &a, hipStream_t st);

// Commit after verification (see spec_commit): byte layout of the cache and the call.
struct CommitArgs {
  uint8_t *kv;
  long layer_stride, half_stride;
  int n_layers, block_size, entry_bytes, max_blocks, n_blocks;
  const int32_t *block_table;
  int32_t *seq_len;
  uint8_t *rec_state;
  const uint8_t *rec_snap;
  long rec_bytes;
  const int32_t *accepted_len;
  const int32_t *verify_len;  // null: Kmax each
  const int32_t *path;        // null: chain
  int B, Kmax;
  int32_t *dev_status;
};
hipError_t launch_commit(const CommitArgs &c, hipStream_t st);

}  // namespace sv
