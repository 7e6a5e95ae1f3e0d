// Commit after verification: the cached target state of the accepted prefix is kept,
// the rest dropped (tutorial page "Let's start over, Misha ...", "The KV cache and
// speculative decoding work together"; Wildberries page, "Why hybrid attention matters
// for speculation" and the n-gram pitfalls, where the linear-attention state went wrong
// across steps with and without a draft).
//
// All of it is data movement, bound by HBM: each request's recurrent state becomes the
// snapshot after its last committed input (rec_bytes read and written), and in a tree
// the accepted path's cache entries move to consecutive positions.  Kernel 1 moves the
// bytes: blocks [0, B * nchunk) copy 64 KiB of one request's state each, the blocks
// after them compact one (request, layer, half) of a tree's cache each.  Kernel 2 then
// advances seq_len, which kernel 1 reads.  Every block validates its request with one
// wave (one lane per depth) and leaves it alone when the commit does not fit.
#include "sv_device.h"

namespace sv {

namespace {

constexpr int CT = 256;                        // threads per block
constexpr int RU = 16;                         // 16-byte pieces per thread of a state copy block
constexpr long REC_CHUNK = (long)CT * 16 * RU;  // state bytes per copy block (64 KiB)
constexpr int MB = 16;                         // cache entries moved per batch

struct CommitReq {
  int A, L, last;  // accepted length, cache length, node of the last committed input
  bool ok;
};

// Request b's commit, checked by the 64 lanes of the calling wave (lane i: depth i).
// With slots != null, lane i <= A also stores the cache slots of the source (node
// path[i]) and destination (depth i) positions.
__device__ CommitReq commit_req(const CommitArgs &c, int b, int lane, long *slots = nullptr) {
  CommitReq r;
  r.A = c.accepted_len[b];
  r.L = c.seq_len[b];
  const int k = c.verify_len ? c.verify_len[b] : c.Kmax;
  const bool ok = r.A >= 0 && r.A <= k && k <= c.Kmax && r.L >= 0;
  bool lane_ok = true;
  int node = lane;
  if (ok && lane <= r.A) {
    const int32_t *pb = c.path ? c.path + (long)b * (c.Kmax + 1) : nullptr;
    node = pb ? pb[lane] : lane;
    const int prev = lane == 0 ? -1 : (pb ? pb[lane - 1] : lane - 1);
    lane_ok = (lane == 0 ? node == 0 : node > prev) && node <= k;
    if (lane_ok && c.n_layers > 0) {
      const long cap = (long)c.max_blocks * c.block_size;
      const long src = (long)r.L + node, dst = (long)r.L + lane;
      lane_ok = src < cap && dst < cap;
      if (lane_ok) {
        const int32_t *row = c.block_table + (long)b * c.max_blocks;
        const int bsrc = row[src / c.block_size], bdst = row[dst / c.block_size];
        lane_ok = bsrc >= 0 && bsrc < c.n_blocks && bdst >= 0 && bdst < c.n_blocks;
        if (slots) {
          slots[2 * lane] = (long)bsrc * c.block_size + src % c.block_size;
          slots[2 * lane + 1] = (long)bdst * c.block_size + dst % c.block_size;
        }
      }
    }
  }
  r.ok = ok && __ballot(!lane_ok) == 0;
  r.last = __shfl(node, ok ? r.A : 0);
  return r;
}

__global__ __launch_bounds__(CT) void k_commit_move(const CommitArgs c, int nchunk, int nrec_blocks) {
  __shared__ CommitReq sreq;
  __shared__ long slots[2 * 64];  // [depth] source and destination cache slots (tree moves)
  const int tid = threadIdx.x;
  const int bid = blockIdx.x;
  const bool rec = bid < nrec_blocks;
  const int q = rec ? bid : bid - nrec_blocks;
  const int b = rec ? q / nchunk : q / (2 * c.n_layers);
  const int part = rec ? q % nchunk : q % (2 * c.n_layers);
  // State copies: the source snapshot follows from A_b (and the path) alone, so its
  // loads are issued before the request is validated, from an index clamped into
  // [0, Kmax] (always in bounds); they are stored only if the commit is valid.
  const long off = (long)part * REC_CHUNK;
  const bool full = rec && c.rec_bytes - off >= REC_CHUNK;
  int guess = 0;
  u32x4 v[RU];
  if (full) {
    guess = min(max(c.accepted_len[b], 0), c.Kmax);
    if (c.path) guess = min(max(c.path[(long)b * (c.Kmax + 1) + guess], 0), c.Kmax);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(
        c.rec_snap + ((long)b * (c.Kmax + 1) + guess) * c.rec_bytes + off);
#pragma unroll
    for (int u = 0; u < RU; ++u) v[u] = __builtin_nontemporal_load(src + u * CT + tid);
  }
  if (tid < 64) {
    const CommitReq r = commit_req(c, b, tid, rec ? nullptr : slots);
    if (tid == 0) sreq = r;
  }
  __syncthreads();
  const CommitReq r = sreq;
  if (!r.ok) return;
  if (rec) {
    const long n = min(REC_CHUNK, c.rec_bytes - off);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(
        c.rec_snap + ((long)b * (c.Kmax + 1) + r.last) * c.rec_bytes + off);
    u32x4 *dst = reinterpret_cast<u32x4 *>(c.rec_state + (long)b * c.rec_bytes + off);
    if (full && guess == r.last) {
#pragma unroll
      for (int u = 0; u < RU; ++u) __builtin_nontemporal_store(v[u], dst + u * CT + tid);
    } else {
      for (long i = tid; i < n / 16; i += CT) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    }
    return;
  }
  // Tree compaction of one (layer, half).  Each thread owns 16-byte pieces of an entry.
  // Depths are moved in batches of MB in increasing order, every source of a batch read
  // before its first write: a source of depth j is node path[j] > path[i] >= i for all
  // earlier depths i, so it is never a destination of this or an earlier batch.
  const int l = part >> 1, h = part & 1;
  uint8_t *base = c.kv + l * c.layer_stride + h * c.half_stride;
  const long eb = c.entry_bytes;
  for (int e = tid * 16; e < c.entry_bytes; e += CT * 16) {
    for (int i0 = 1; i0 <= r.A; i0 += MB) {
      u32x4 v[MB];
#pragma unroll
      for (int g = 0; g < MB; ++g) {
        const int i = i0 + g;
        if (i <= r.A && slots[2 * i] != slots[2 * i + 1])
          v[g] = *reinterpret_cast<const u32x4 *>(base + slots[2 * i] * eb + e);
      }
#pragma unroll
      for (int g = 0; g < MB; ++g) {
        const int i = i0 + g;
        if (i <= r.A && slots[2 * i] != slots[2 * i + 1])
          *reinterpret_cast<u32x4 *>(base + slots[2 * i + 1] * eb + e) = v[g];
      }
    }
  }
}

// One wave per request: the new cache length, or the status of a commit that did not fit.
__global__ __launch_bounds__(CT) void k_commit_len(const CommitArgs c) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (CT / 64) + (threadIdx.x >> 6);
  if (b >= c.B) return;
  const CommitReq r = commit_req(c, b, lane);
  if (lane == 0) {
    if (r.ok) c.seq_len[b] = r.L + r.A + 1;
    else if (r.A >= 0 && c.dev_status) atomicCAS(c.dev_status, SV_DEV_OK, SV_DEV_BAD_COMMIT);
  }
}

}  // namespace

hipError_t launch_commit(const CommitArgs &c, hipStream_t st) {
  const long nchunk = c.rec_bytes > 0 ? (c.rec_bytes + REC_CHUNK - 1) / REC_CHUNK : 0;
  const long nrec = nchunk * c.B;
  const long nkv = (c.path && c.n_layers > 0) ? (long)c.B * 2 * c.n_layers : 0;
  if (nrec + nkv > 0x7fffffffL) return hipErrorInvalidValue;
  if (nrec + nkv > 0) {
    hipLaunchKernelGGL(k_commit_move, dim3((unsigned)(nrec + nkv)), dim3(CT), 0, st, c, (int)nchunk, (int)nrec);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_commit_len, dim3((unsigned)((c.B + CT / 64 - 1) / (CT / 64))), dim3(CT), 0, st, c);
  return hipGetLastError();
}

}  // namespace sv
