/*
 * spec_verify.h -- C ABI of libspecverify, the draft-block verification step of
 * speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * One call scores the K draft tokens of each of B requests plus a bonus position
 * in a single pass over the weights of the target's final SwiGLU MLP and its LM
 * head, then runs the acceptance rule over the full vocabulary.
 *
 * The operation (sources are cited by page title and section):
 *  - "Speculative decoding in production: comparing methods in the Wildberries
 *    shopping assistant", "Where speculative decoding came from": one target pass
 *    scores every draft token; the longest correct prefix is accepted and the
 *    target's own token is put at the first error.  "A bit of theory", Statement 1:
 *    a draft token x is accepted with probability min(1, p(x)/q(x)), where p is the
 *    target distribution after temperature and q the draft's; on rejection a token
 *    is drawn from the normalised remainder max(0, p - q).
 *  - "Let's start over, Misha: speculative decoding from draft to verification",
 *    "How it works": when every draft token passes, the same pass yields one more
 *    target token; "Why isn't the answer spoiled?": at temperature 0 the check
 *    is an argmax comparison.
 *  - "DSpark: speculative decoding with confidence-scheduled verification and
 *    semi-autoregressive generation": each request's verify length is chosen from
 *    the estimated survival probability of its draft prefix under the engine's
 *    capacity.
 *
 * Model of the scored tail (one reading where the pages are silent): for every
 * target row, a = bf16(silu(h W_gate^T) * (h W_up^T)), y = bf16(h + a W_down^T),
 * target logits z = y W_lm^T; draft logits are h_draft W_lm^T with the same
 * (shared) LM head.  With d_ff == 0 there is no MLP and y = h.
 *
 * Conventions for every entry point
 *  - All array pointers are DEVICE pointers owned by the caller; the library never
 *    allocates, frees or keeps them.  Weights and hidden rows must be 16-byte
 *    aligned.  bf16 values are passed as their uint16_t bit patterns.  Arrays are
 *    dense and row-major; weights are [out, in].
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work; outputs are valid once the stream has passed the call.  There is no
 *    host synchronisation inside a call.  Concurrent calls are safe if they use
 *    distinct workspaces and outputs.
 *  - `ws` is caller-provided device scratch of at least sv_workspace_bytes(...)
 *    bytes, 256-byte aligned.  Its contents on entry do not matter.
 *  - Row order: request b, position j is row b*(K+1)+j of `h` ([B, K+1, d]) and
 *    row b*K+j of `h_draft` / `draft` ([B, K, ...]).  Target row j scores draft
 *    token j+1 (draft[b*K+j]); target row K is the bonus position.
 *  - Coins `u` [B, K+1] are fp32 in [0, 1): u[b, j] (j < K) is the acceptance coin
 *    of draft token j+1; u[b, K] is the single coin of the final (residual or
 *    bonus) sample.  In scheduled mode K is Kmax and the final coin is u[b, Kmax].
 *  - Return value: SV_OK, or a negative SV_E* code; nothing is enqueued when the
 *    arguments are rejected.  Data errors only visible on the device (a draft id
 *    outside [0, V), a non-finite row statistic) set *dev_status to the first
 *    SV_DEV_* code seen and make that request's outputs -1.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_OK 0
#define SV_EINVAL (-1)      /* bad sizes, NULL required pointer, misalignment, T <= 0, budget < B */
#define SV_MAX_K 8190       /* largest K (Kmax) of a greedy, sampled or scheduled call */
#define SV_EWORKSPACE (-2)  /* ws_bytes smaller than sv_workspace_bytes() */
#define SV_EHIP (-3)        /* a HIP launch or runtime call failed */
#define SV_ESCRATCH (-4)    /* spec_verify_sample_noalloc: the sizes need more than SV_STATIC_SCRATCH_BYTES */

#define SV_DEV_OK 0
#define SV_DEV_BAD_TOKEN 1  /* a draft id outside [0, V) */
#define SV_DEV_NONFINITE 2  /* a row statistic (max or log-sum-exp) is not finite */

#define SV_MODE_GREEDY 0
#define SV_MODE_SAMPLE 1
#define SV_MODE_SCHEDULED 2
#define SV_MODE_PROPOSE 3

/* Per-row diagnostic record (floats), written when sv_outputs.diag != NULL:
 * [0] log-sum-exp of z/T (greedy: T = 1)   [1] argmax (lowest index, as float)
 * [2] top-1 minus top-2 logit (z units)    [3] max logit
 * [4] logit of the row's draft token (NaN on bonus rows / when unused)
 * [5] probability of that token: p(x) on target rows, q(x) on draft rows
 * [6] acceptance ratio p(x)/q(x) (target rows), top-1 probability (draft rows)
 * [7] reserved (0) */
#define SV_DIAG_COLS 8

#define SV_WEIGHTS_BF16 0     /* bf16 weights (uint16 bit patterns) */
#define SV_WEIGHTS_FP8_E4M3 1 /* 8-bit E4M3 codes (uint8) with one fp32 scale per output row */

/* Weights, row-major [out, in].  FP8 weights (reading of the pages' FP8 serving: the
 * OCP 8-bit E4M3 format, one fp32 scale per output row, bf16 activations) stand for
 * decode(code) * scale[row] and are supported when every product of the call streams
 * its weights (at most 16 target rows with an MLP, at most 32 rows through the LM
 * head, e.g. one 16-token block); other calls return SV_EINVAL, and
 * sv_workspace_bytes returns 0 for them. */
typedef struct sv_weights {
  const void *w_gate; /* [d_ff, d]; NULL iff d_ff == 0 */
  const void *w_up;   /* [d_ff, d]; NULL iff d_ff == 0 */
  const void *w_down; /* [d, d_ff]; NULL iff d_ff == 0 */
  const void *w_lm;   /* [V, d] shared LM head */
  int32_t d;          /* hidden size, multiple of 64 */
  int32_t d_ff;       /* MLP width, multiple of 64, or 0 */
  int32_t V;          /* vocabulary, 1 <= V <= 524288 */
  int32_t wtype;      /* SV_WEIGHTS_*; 0 (bf16) when the struct is zero-initialised */
  const float *s_gate; /* FP8: [d_ff] scales of w_gate rows (else ignored) */
  const float *s_up;   /* FP8: [d_ff] */
  const float *s_down; /* FP8: [d] */
  const float *s_lm;   /* FP8: [V] */
} sv_weights;

typedef struct sv_outputs {
  int32_t *accepted_len; /* [B] required: A_b, accepted draft tokens (-1 on a bad request) */
  int32_t *emitted;      /* [B, K+1] required: first A_b+1 entries valid, the rest -1 */
  int32_t *verify_len;   /* [B] scheduled mode: k_b drafts verified; may be NULL */
  float *tau;            /* [1] required: mean over requests of A_b + 1 */
  int64_t *counters;     /* [3] accepted drafts, verified drafts, emitted tokens; may be NULL */
  int32_t *dev_status;   /* [1] SV_DEV_* code; may be NULL */
  float *diag;           /* per-row SV_DIAG_COLS records; may be NULL.  Rows: target rows
                            [B*(K+1)] then draft rows [B*K] (greedy: target rows only) */
  float *logits;         /* fp32 logits, same row order as diag, [rows, V]; may be NULL.
                            Scheduled mode writes only the verified target rows */
  uint16_t *hidden;      /* bf16 MLP output y [B*(K+1), d]; may be NULL; written only when
                            d_ff > 0 (scheduled mode: verified rows only) */
  void *ev_lm_begin;     /* optional hipEvent_t pair recorded on `stream` right before and */
  void *ev_lm_end;       /* after the dominant LM-head GEMM (scheduled mode: the draft-row
                            pass); both NULL to skip.  For measurement only. */
} sv_outputs;

/* Bytes of device workspace a call with these sizes needs (0 on invalid sizes).  The pages
 * define no memory plan; this is the library's own (fp32 logit rows for the sampled modes,
 * per-row statistic records, MLP activations).
 * mode: SV_MODE_*; K is Kmax in scheduled mode (the size covers any budget); in
 * propose mode B is the number of draft rows and K is ignored. */
size_t sv_workspace_bytes(int mode, int B, int K, const sv_weights *w);

/* Greedy verification (temperature 0).  Source: "Let's start over, Misha", "Why isn't the
 * answer spoiled?" (at temperature 0 a draft token is kept when it is the target's argmax)
 * and the Wildberries page, "Where speculative decoding came from" (the longest correct
 * prefix is kept and the target's own token is put at the first error; one pass scores
 * every position).  h: [B, K+1, d] bf16 target hidden rows;
 * draft: [B, K] int32.  A_b is the first j with draft[b, j] != argmax of target row
 * j (K if none); the emitted tokens are draft[b, 0..A_b-1] then the argmax of row
 * A_b.  Ties in the argmax go to the lowest index.  The diag records use T = 1. */
int spec_verify_greedy(const sv_weights *w, const uint16_t *h, const int32_t *draft, int B, int K,
                       void *ws, size_t ws_bytes, sv_outputs *out, void *stream);

/* Rejection-sampling verification at temperature T > 0.  Source: the Wildberries page, "A
 * bit of theory", Statement 1 (accept x with probability min(1, p(x)/q(x)), p and q after
 * temperature; on rejection draw from the normalised max(0, p - q)), Statement 2 (the
 * accepted length and tau), and "Let's start over, Misha", "How it works" (when every draft
 * passes the same pass yields one more token from p).  h: [B, K+1, d];
 * h_draft: [B, K, d] draft hidden rows scored by the same LM head; draft: [B, K];
 * u: [B, K+1].  Draft token j+1 is accepted while u[b, j] < p_j(x)/q_j(x); at the
 * first rejection the emitted token is drawn from max(0, p_j - q_j) (falling back to
 * p_j if that is all zero) and when all K pass, from p_K, both by inverse CDF over
 * ascending token ids with the coin u[b, K]. */
int spec_verify_sample(const sv_weights *w, const uint16_t *h, const uint16_t *h_draft,
                       const int32_t *draft, const float *u, float T, int B, int K, void *ws,
                       size_t ws_bytes, sv_outputs *out, void *stream);

/* Bytes of device scratch held by the library on each GPU it runs on (until the process ends). */
#define SV_STATIC_SCRATCH_BYTES (32u << 20)

/* spec_verify_sample for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same computation and
 * the same kernels, with the workspace taken from a static device array of
 * SV_STATIC_SCRATCH_BYTES bytes per GPU instead of the caller's `ws`.  The caller still
 * passes inputs and outputs.  Calls whose sizes need more workspace than that
 * (sv_workspace_bytes(SV_MODE_SAMPLE, B, K, w) > SV_STATIC_SCRATCH_BYTES) return
 * SV_ESCRATCH and enqueue nothing; e.g. one 16-token block (B = 1, K = 15, d = 4096,
 * V = 151936) needs about 18.6 MiB.  No HIP allocation or free is made; the first call on
 * a device looks up the array's address there.  All calls on one GPU share its array, so
 * calls that overlap on one GPU (different streams or threads without ordering) race:
 * order them on one stream.  The array's contents on entry do not matter. */
int spec_verify_sample_noalloc(const sv_weights *w, const uint16_t *h, const uint16_t *h_draft,
                               const int32_t *draft, const float *u, float T, int B, int K, sv_outputs *out,
                               void *stream);

/* Confidence-scheduled verification at temperature T > 0.  Source: "DSpark: speculative
 * decoding with confidence-scheduled verification and semi-autoregressive generation" (each
 * request's verify length follows the estimated survival probability of its draft prefix,
 * under the engine's capacity); the rule below is the library's reading of it (the page
 * gives the idea, not the formula), then the sampled rule of spec_verify_sample.  Shapes as in
 * spec_verify_sample with K = Kmax.  The LM head first scores all B*Kmax draft rows;
 * c[b, k] = max_v q_{b,k}(v), survival s_b(k) = prod_{i<=k} c[b, i].  Positions with
 * s_b(k) >= survival_threshold are eligible; each request always verifies its own
 * target row, and when B + #eligible > budget_rows only the budget_rows - B eligible
 * positions with the largest floor(1024 * s) are kept (ties: lower request, then lower
 * position).  Request b then runs the sampled rule on its first k_b drafts, with
 * u[b, 0..k_b-1] and the final coin u[b, Kmax].  Requires budget_rows >= B and
 * 0 < survival_threshold <= 1, B <= 8192 and B*Kmax <= 8192.  verify_len (if given)
 * receives k_b. */
int spec_verify_scheduled(const sv_weights *w, const uint16_t *h, const uint16_t *h_draft,
                          const int32_t *draft, const float *u, float T, float survival_threshold,
                          int budget_rows, int B, int Kmax, void *ws, size_t ws_bytes,
                          sv_outputs *out, void *stream);

/* The drafter's step on the shared LM head: the call before verification in MTP/EAGLE-style
 * drafting ("Speculative decoding in vLLM and SGLang ...", "EAGLE and EAGLE-3": a light head
 * over the target's hidden states proposes the next tokens; that it ends in the target's own
 * LM head is this library's reading).  h_draft: [rows, d]; coins: [rows] (unused when T == 0).
 * draft_out[r] = token drawn from q = softmax(h_draft[r] W_lm^T / T) by inverse CDF
 * with coins[r], or the argmax when T == 0; conf_out[r] (may be NULL) = max_v q(v)
 * (1 when T == 0). */
int spec_draft_propose(const sv_weights *w, const uint16_t *h_draft, const float *coins, float T,
                       int rows, void *ws, size_t ws_bytes, int32_t *draft_out, float *conf_out,
                       void *stream);

#define SV_DEV_BAD_TREE 4 /* spec_verify_tree: a parent index outside [0, j] for node j+1 */
#define SV_DEV_TIMEOUT 5  /* spec_verify_tree: the blocks of a request never met (outputs -1) */

/* Tree (multi-candidate) verification ("Let's start over, Misha ...", "EAGLE" and
 * "Medusa": candidate trees checked by the target in one pass with tree attention;
 * "Speculative decoding in vLLM and SGLang ...": draft steps, top-k candidates per step
 * and a verification token budget).  The pages give no acceptance rule for a tree; this
 * one is Statement 1 of the Wildberries page applied to a node's candidates in turn.
 *
 * Each request verifies a tree of K+1 nodes: node 0 is the last emitted token; node j+1
 * (j < K) carries draft token tokens[b, j] and has parent parent[b, j] in [0, j].
 * h: [B, K+1, d] target hidden rows per node (after tree attention over the node's root
 * path); h_draft: [B, K, d] drafter rows of nodes 0..K-1 (T > 0 only), whose distribution
 * q_u produced the children of node u.
 *  - T == 0 (greedy): from node 0, move to the lowest-index child whose token is the
 *    target argmax at the current node; where no child matches, emit that argmax.
 *  - T > 0: the children c of the current node u are tested in index order; c (token x)
 *    passes when u[b, c-1] < r(x) / q_u(x), where r = p_u at first and, after each failed
 *    child, the normalised max(0, r - q_u) (p_u again if that is all zero).  The first
 *    child that passes becomes the current node; when none passes, or u has no children,
 *    the emitted token is drawn from r by inverse CDF over ascending ids with u[b, K].
 * accepted_len[b] = depth reached; emitted[b, 0..A] = tokens of the path's nodes, then
 * the final token; path (may be NULL) [B, K+1] = node at each depth, -1 beyond A (the
 * tree path spec_commit takes).  A chain (parent[b, j] = j) gives exactly the results of
 * spec_verify_greedy / spec_verify_sample.  diag rows: target rows then (T > 0) draft
 * rows, records [0..3] as above, [4..6] NaN.  At T > 0 the residual passes of a request may
 * run on several workgroups that meet at a device-side counter; wait_polls bounds how often
 * a workgroup polls for the others per meeting (< 0: 65,536, about 65 ms; 0 makes every
 * meeting fail, which tests the time-out path): a request whose workgroups never meet gets
 * SV_DEV_TIMEOUT and outputs -1 instead of a hang.  Requires K <= 63.  Workspace:
 * sv_workspace_bytes(SV_MODE_GREEDY, B, K, w) at T == 0, SV_MODE_SAMPLE at T > 0.  A bad
 * parent sets SV_DEV_BAD_TREE, a token outside [0, V) SV_DEV_BAD_TOKEN (request outputs -1). */
int spec_verify_tree(const sv_weights *w, const uint16_t *h, const uint16_t *h_draft, const int32_t *tokens,
                     const int32_t *parent, const float *u, float T, int B, int K, void *ws, size_t ws_bytes,
                     sv_outputs *out, int32_t *path, int wait_polls, void *stream);

/* Cached target state of B requests, for the commit after a verify call.
 *
 * Paged KV cache of the attention layers: the entry (entry_bytes bytes) of position p
 * of request b in layer l, half h (0 = keys, 1 = values) starts at
 *   kv + l * layer_stride + h * half_stride
 *      + (block_table[b * max_blocks + p / block_size] * block_size + p % block_size) * entry_bytes.
 * Recurrent states (linear-attention layers, short convolutions, ...) are opaque bytes:
 * rec_state [B, rec_bytes] is the state each request carries between steps and
 * rec_snap [B, Kmax+1, rec_bytes] holds, for each input j of the last verify block,
 * the state after that input (written by the target's forward, outside this library).
 * rec_state and rec_snap must not overlap. */
typedef struct sv_cache {
  void *kv;                    /* NULL iff n_layers == 0; 16-byte aligned */
  int64_t layer_stride;        /* bytes, multiple of 16 */
  int64_t half_stride;         /* bytes, multiple of 16 */
  int32_t n_layers;            /* attention layers with a KV cache (0: none) */
  int32_t block_size;          /* tokens per cache block, >= 1 */
  int32_t entry_bytes;         /* bytes of one token's keys (or values) in one layer, multiple of 16 */
  int32_t max_blocks;          /* columns of block_table */
  int32_t n_blocks;            /* blocks in the pool: ids in block_table lie in [0, n_blocks) */
  const int32_t *block_table;  /* [B, max_blocks] block ids */
  int32_t *seq_len;            /* [B] required: tokens in each request's cache; advanced by a commit */
  void *rec_state;             /* [B, rec_bytes], 16-byte aligned; NULL iff rec_bytes == 0 */
  const void *rec_snap;        /* [B, Kmax+1, rec_bytes], 16-byte aligned; NULL iff rec_bytes == 0 */
  int64_t rec_bytes;           /* multiple of 16, or 0 */
} sv_cache;

#define SV_DEV_BAD_COMMIT 3 /* spec_commit: an accepted length or path that does not fit its block */

/* Commit after verification: keep the cached state of the accepted prefix only
 * ("Let's start over, Misha ...", "The KV cache and speculative decoding work together":
 * the target keeps state for the accepted part of the block and drops the rejected
 * tail; "Speculative decoding in production ...", "Why hybrid attention matters for
 * speculation" and the n-gram pitfalls: the linear-attention state must follow the
 * committed tokens on steps with and without a draft).
 *
 * The verify block of request b had k_b + 1 inputs (the last emitted token, then k_b
 * drafts; k_b = verify_len[b], or Kmax when verify_len is NULL; k_b = 0 is a step
 * without a draft) whose keys/values the target wrote at positions seq_len[b] + j.
 * With A_b = accepted_len[b] (from a verify call), inputs 0..A_b are committed:
 *  - chain (path == NULL): the entries stay where they are; seq_len[b] += A_b + 1;
 *  - tree (path != NULL, [B, Kmax+1]): node path[b, i] is the accepted node at depth i
 *    (path[b, 0] = 0, strictly increasing, <= k_b); its entries, written at
 *    seq_len[b] + path[b, i], move to seq_len[b] + i in every layer and both halves;
 *  - rec_state[b] = rec_snap[b, n] with n = A_b (chain) or path[b, A_b] (tree).
 * Requests with A_b < 0 (flagged by the verify call) are left unchanged.  A request whose
 * A_b > k_b, whose path is not as above, or whose touched positions (seq_len[b] + i and
 * seq_len[b] + path[b, i] for i <= A_b) run past its block-table row or map to block ids
 * outside the pool (checked only when n_layers > 0) is left unchanged
 * and sets *dev_status (may be NULL; only written while it holds SV_DEV_OK, so a verify
 * call's code is kept) to SV_DEV_BAD_COMMIT.  Entries beyond the new seq_len keep stale
 * bytes.  Requires 0 <= Kmax <= 63.  Two kernels on `stream`; no workspace. */
int spec_commit(const sv_cache *c, const int32_t *accepted_len, const int32_t *verify_len,
                const int32_t *path, int B, int Kmax, int32_t *dev_status, void *stream);

/* Library version string, a text for an SV_E* code, and the HIP error text behind
 * the last SV_EHIP returned on the calling thread. */
const char *sv_version(void);
const char *sv_strerror(int code);
const char *sv_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
