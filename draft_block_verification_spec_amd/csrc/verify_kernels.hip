// Acceptance, sampling, scheduling and bookkeeping kernels of the verification step.
//
// Rules implemented (page titles and sections):
//  * Wildberries page, "A bit of theory", Statement 1: draft token x passes with
//    probability min(1, p(x)/q(x)), with p and q taken after temperature; at the
//    first rejection the token is drawn from the normalised max(0, p - q).
//  * "Let's start over, Misha", "How it works": tokens are checked left to right;
//    when all K pass the bonus token comes from the same pass.  "Why isn't the
//    answer spoiled?": at temperature 0 the check is an argmax match.
//  * DSpark summary page: the verify length of each request follows the
//    estimated survival probability of its draft prefix, under a capacity budget.
#include <atomic>
#include "sv_device.h"

namespace sv {

namespace {

constexpr int NT = 256;  // threads per block for the small kernels
constexpr int PER = 8;   // tokens per thread and chunk in the chunk-sum kernel (a chunk is at most NT * PER = 2048)

__device__ void set_status(int32_t *st, int code) {
  if (st) atomicCAS(st, 0, code);
}

// Merge the nslots partials of one row with one wave; result valid in every lane.  Each
// lane merges slots lane, lane + 64, ... in order; their loads are issued in batches of
// BATCH ahead of the merges, so a row of ~1200 partials costs 2 memory round trips with
// BATCH = 12 (3 with 8), not 19.
template <int BATCH = 8>
__device__ StatPart wave_merge_row(const StatPart *parts, int nslots, float invT, bool want_s) {
  const int lane = threadIdx.x & 63;
  StatPart st = stat_empty();
  for (int i0 = 0; i0 < nslots; i0 += 64 * BATCH) {
    StatPart p[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int i = i0 + 64 * k + lane;
      p[k] = i < nslots ? parts[i] : stat_empty();
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) st = stat_merge(st, p[k], invT, want_s);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) st = stat_merge(st, stat_shfl_xor(st, off), invT, want_s);
  return st;
}

__global__ void k_init(int32_t *z, long n, int32_t *dev_status) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) z[i] = 0;
  if (dev_status && blockIdx.x == 0 && threadIdx.x == 0) *dev_status = 0;
}

// ---- block-wide helpers (fixed reduction order: results do not depend on timing)
__device__ float block_sum(float v, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  return t;
}

__device__ int block_min_int(int v, int *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) t = min(t, red[w]);
  return t;
}

// Inclusive prefix sum over the block in thread order: shuffle scan inside each wave,
// then the wave totals (fixed order).  buf needs one float per wave.
__device__ float block_incl_scan(float v, float *buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float x = __shfl_up(v, off);
    if (lane >= off) v += x;
  }
  __syncthreads();
  if (lane == 63) buf[wave] = v;
  __syncthreads();
  float base = 0.f;
  for (int w = 0; w < wave; ++w) base += buf[w];
  return base + v;
}

// End-of-call bookkeeping: tau = mean(A_b + 1) over valid requests and the counters.
__device__ void finalize_block(const FinalizeArgs &f) {
  __shared__ long long red[4][16];
  long long sa = 0, sd = 0, se = 0, nv = 0;
  for (int b = threadIdx.x; b < f.B; b += blockDim.x) {
    const int A = f.acc[b];
    if (A < 0) continue;
    sa += A;
    sd += f.vlen ? f.vlen[b] : f.K;
    se += A + 1;
    nv += 1;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    sa += __shfl_xor(sa, off);
    sd += __shfl_xor(sd, off);
    se += __shfl_xor(se, off);
    nv += __shfl_xor(nv, off);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[0][wave] = sa; red[1][wave] = sd; red[2][wave] = se; red[3][wave] = nv; }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long ta = 0, td = 0, te = 0, valid = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) { ta += red[0][w]; td += red[1][w]; te += red[2][w]; valid += red[3][w]; }
    *f.tau = valid ? (float)((double)te / (double)valid) : 0.f;
    if (f.counters) { f.counters[0] = ta; f.counters[1] = td; f.counters[2] = te; }
  }
}

// Is this block the last one to arrive at `counter` (of `total`)?  Release before, acquire after.
__device__ bool arrive_last(int32_t *counter, int total, int *flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const int old = atomicAdd(counter, 1);
    *flag = (old == total - 1);
  }
  __syncthreads();
  const bool last = *flag != 0;
  if (last) __threadfence();
  return last;
}

// One block per request.  Row statistics are merged by one wave per row.
__global__ __launch_bounds__(1024) void k_accept_sample(const AcceptArgs a) {
  extern __shared__ float sm[];
  const int b = blockIdx.x;
  const int Kmax = a.K;
  const int Kb = a.verify_len ? a.verify_len[b] : Kmax;
  const long trow0 = a.row_off ? a.row_off[b] : (long)b * (Kmax + 1);
  const long drow0 = (long)b * Kmax;
  const int nslots_t = a.nslots_t_dev ? *a.nslots_t_dev : a.nslots_t;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float *lse_t = sm;                  // [Kmax+1]
  float *lse_d = sm + (Kmax + 1);     // [Kmax]
  __shared__ int bad;
  if (threadIdx.x == 0) {
    bad = 0;
    a.job_cnt[b] = 0;  // arrival counters of the sampling kernel that follows
    if (b == 0) *a.done_cnt = 0;
  }
  __syncthreads();
  const int nw = blockDim.x >> 6;
  // wave 0: the inputs of the first 64 acceptance decisions, loaded ahead of the
  // statistics (the logits at the draft token do not depend on the normalisers)
  int x0 = 0;
  float u0 = 0.f, zt0 = 0.f, zd0 = 0.f;
  if (wave == 0 && lane < Kb) {
    x0 = a.draft[drow0 + lane];
    u0 = a.u[(long)b * (Kmax + 1) + lane];
    if (x0 >= 0 && x0 < a.V) {
      zt0 = a.logits_t[(trow0 + lane) * (long)a.V + x0];
      zd0 = a.logits_d[(drow0 + lane) * (long)a.V + x0];
    }
  }

  // row statistics: target rows 0..Kb, draft rows 0..Kb-1
  const int nrows = 2 * Kb + 1;
  for (int r = wave; r < nrows; r += nw) {
    const bool is_t = r <= Kb;
    const int j = is_t ? r : r - Kb - 1;
    const StatPart *pp = is_t ? a.parts_t + (trow0 + j) * nslots_t : a.parts_d + (drow0 + j) * a.nslots_d;
    const StatPart st = wave_merge_row<12>(pp, is_t ? nslots_t : a.nslots_d, a.invT, true);
    const float lse = st.b1 * a.invT + __logf(st.s);
    if (lane == 0) {
      if (is_t) lse_t[j] = lse; else lse_d[j] = lse;
      if (!isfinite(lse)) bad = SV_DEV_NONFINITE;
      if (a.diag) {
        const long drow = is_t ? (long)b * (Kmax + 1) + j : (long)a.B * (Kmax + 1) + drow0 + j;
        float *dg = a.diag + drow * SV_DIAG_COLS;
        dg[0] = lse; dg[1] = (float)st.i1; dg[2] = st.b1 - st.b2; dg[3] = st.b1;
        dg[4] = NAN; dg[5] = NAN; dg[6] = is_t ? NAN : 1.f / st.s; dg[7] = 0.f;
      }
    }
  }
  __syncthreads();

  // acceptance decisions: lane j of wave 0 handles draft position j+1
  if (wave == 0) {
    bool ok = true;
    int A = 0;
    bool rej = false;
    for (int base = 0; base < Kb; base += 64) {
      const int j = base + lane;
      bool acc = false, bad_tok = false;
      if (j < Kb) {
        const int x = base == 0 ? x0 : a.draft[drow0 + j];
        if (x < 0 || x >= a.V) {
          bad_tok = true;
        } else {
          const float zt = base == 0 ? zt0 : a.logits_t[(trow0 + j) * (long)a.V + x];
          const float zd = base == 0 ? zd0 : a.logits_d[(drow0 + j) * (long)a.V + x];
          const float lpt = zt * a.invT - lse_t[j];
          const float lqd = zd * a.invT - lse_d[j];
          const float ratio = __expf(lpt - lqd);
          const float u = base == 0 ? u0 : a.u[(long)b * (Kmax + 1) + j];
          acc = u < ratio;
          if (a.diag) {
            float *dt = a.diag + ((long)b * (Kmax + 1) + j) * SV_DIAG_COLS;
            dt[4] = zt; dt[5] = __expf(lpt); dt[6] = ratio;
            float *dd = a.diag + ((long)a.B * (Kmax + 1) + drow0 + j) * SV_DIAG_COLS;
            dd[4] = zd; dd[5] = __expf(lqd);
          }
        }
      }
      if (__any(bad_tok)) ok = false;
      if (!rej) {
        const unsigned long long live = (Kb - base >= 64) ? ~0ull : ((1ull << (Kb - base)) - 1ull);
        const unsigned long long rejm = __ballot(!acc) & live;
        if (rejm) {
          A = base + __ffsll((long long)rejm) - 1;
          rej = true;
        } else {
          A = min(Kb, base + 64);
        }
      }
    }
    if (lane == 0) {
      if (!ok) set_status(a.dev_status, SV_DEV_BAD_TOKEN);
      if (bad) set_status(a.dev_status, bad);
      const bool good = ok && !bad;
      a.accepted_len[b] = good ? A : -1;
      SampleJob jb;
      jb.u = a.u[(long)b * (Kmax + 1) + Kmax];
      jb.lse1 = lse_t[A];
      jb.z1 = a.logits_t + (trow0 + A) * (long)a.V;
      if (A < Kb) {
        jb.z2 = a.logits_d + (drow0 + A) * (long)a.V;
        jb.lse2 = lse_d[A];
      } else {
        jb.z2 = nullptr;
        jb.lse2 = 0.f;
      }
      jb.out_index = good ? b * (Kmax + 1) + A : -1;
      a.jobs[b] = jb;
    }
    for (int j = lane; j <= Kmax; j += 64) {
      int v = -1;
      if (ok && !bad && j < A) v = a.draft[drow0 + j];
      a.emitted[(long)b * (Kmax + 1) + j] = v;  // position A is written by the sampler
    }
  }
}

__global__ __launch_bounds__(1024) void k_accept_greedy(const AcceptArgs a) {
  extern __shared__ float sm[];
  int *amax = reinterpret_cast<int *>(sm);  // [K+1]
  const int b = blockIdx.x, K = a.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long trow0 = (long)b * (K + 1);
  __shared__ int bad, flag;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int nw = blockDim.x >> 6;
  // draft tokens of the first 64 positions, loaded ahead of the statistics
  const int x0 = (wave == 0 && lane < K) ? a.draft[(long)b * K + lane] : -1;
  auto finish_row = [&](int j, const StatPart &st) {
    amax[j] = st.i1;
    if (!isfinite(st.b1)) bad = SV_DEV_NONFINITE;
    if (a.diag) {
      float *dg = a.diag + (trow0 + j) * SV_DIAG_COLS;
      dg[0] = st.b1 + __logf(st.s); dg[1] = (float)st.i1; dg[2] = st.b1 - st.b2; dg[3] = st.b1;
      dg[4] = NAN; dg[5] = NAN; dg[6] = NAN; dg[7] = 0.f;
    }
  };
  if (2 * (K + 1) <= nw) {
    // two waves per row, each merging half of its partials (one round of loads for ~1200
    // partials), the halves combined in a fixed order
    __shared__ StatPart halves[2][8];
    const int j = wave % (K + 1), h = wave / (K + 1);
    if (h < 2) {
      const int half = (a.nslots_t + 1) / 2;
      const int s0 = h * half, n = min(a.nslots_t, s0 + half) - s0;
      const StatPart st = wave_merge_row<12>(a.parts_t + (trow0 + j) * a.nslots_t + s0, n, 1.f, a.diag != nullptr);
      if (lane == 0) halves[h][j] = st;
    }
    __syncthreads();
    if (wave <= K && lane == 0) finish_row(wave, stat_merge(halves[0][wave], halves[1][wave], 1.f, a.diag != nullptr));
  } else {
    for (int j = wave; j <= K; j += nw) {
      const StatPart st = wave_merge_row<12>(a.parts_t + (trow0 + j) * a.nslots_t, a.nslots_t, 1.f, a.diag != nullptr);
      if (lane == 0) finish_row(j, st);
    }
  }
  __syncthreads();
  if (wave == 0) {
    bool ok = true, rej = false;
    int A = 0;
    for (int base = 0; base < K; base += 64) {
      const int j = base + lane;
      bool match = false;
      if (j < K) {
        const int x = base == 0 ? x0 : a.draft[(long)b * K + j];
        if (x < 0 || x >= a.V) ok = false;
        match = (x == amax[j]);
        if (a.diag && x >= 0 && x < a.V && a.logits_t) a.diag[(trow0 + j) * SV_DIAG_COLS + 4] = a.logits_t[(trow0 + j) * (long)a.V + x];
      }
      if (!rej) {
        const unsigned long long live = (K - base >= 64) ? ~0ull : ((1ull << (K - base)) - 1ull);
        const unsigned long long mis = __ballot(!match) & live;
        if (mis) { A = base + __ffsll((long long)mis) - 1; rej = true; }
        else A = min(K, base + 64);
      }
    }
    const bool allok = !__any(!ok);
    const bool good = allok && !bad;
    if (lane == 0) {
      if (!allok) set_status(a.dev_status, SV_DEV_BAD_TOKEN);
      if (bad) set_status(a.dev_status, bad);
      a.accepted_len[b] = good ? A : -1;
    }
    for (int j = lane; j <= K; j += 64) {
      int v = -1;
      if (good && j < A) v = j < 64 ? x0 : a.draft[(long)b * K + j];
      if (good && j == A) v = amax[A];
      a.emitted[(long)b * (K + 1) + j] = v;
    }
    if (a.B == 1 && a.fin.acc && lane == 0) {
      // a single request: the bookkeeping needs no other block
      *a.fin.tau = good ? (float)(A + 1) : 0.f;
      if (a.fin.counters) {
        a.fin.counters[0] = good ? A : 0;
        a.fin.counters[1] = good ? K : 0;
        a.fin.counters[2] = good ? A + 1 : 0;
      }
    }
  }
  if (a.B > 1 && a.fin.acc && arrive_last(a.done_cnt, a.B, &flag)) finalize_block(a.fin);
}

constexpr int SUBS = 5;  // sampling chunks per block of the chunk-sum kernel

// Inclusive prefix sum over the 64 lanes of a wave, in lane order.
__device__ __forceinline__ float wave_incl_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float x = __shfl_up(v, off);
    if (lane >= off) v += x;
  }
  return v;
}

// Position of a draw inside a sequence held by the lanes of a wave in lane order.
// Lane l holds the weights w[0..n) of consecutive items starting at item0 (n <= NI),
// incl is the wave's inclusive prefix sum of the lane totals, base the sum of all items
// before the sequence.  Returns (in every lane) the first item whose running sum
// exceeds target; if rounding leaves none, the last item of positive weight; if no
// item has weight, item0 of lane 0.  *run_before gets the running sum before that item.
template <int NI>
__device__ int wave_find(const float (&w)[NI], int n, int item0, float base, float incl, float lane_tot,
                         float target, float *run_before) {
  float run = base + incl - lane_tot;
  int hit = -1, last = -1;
  float hit_run = 0.f, last_run = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i < n && w[i] > 0.f) {
      if (hit < 0 && run + w[i] > target) {
        hit = item0 + i;
        hit_run = run;
      }
      last = item0 + i;
      last_run = run;
    }
    if (i < n) run += w[i];
  }
  const unsigned long long mh = __ballot(hit >= 0);
  if (mh) {
    const int src = __ffsll((long long)mh) - 1;
    *run_before = __shfl(hit_run, src);
    return __shfl(hit, src);
  }
  const unsigned long long ml = __ballot(last >= 0);
  if (ml) {
    const int src = 63 - __clzll((long long)ml);
    *run_before = __shfl(last_run, src);
    return __shfl(last, src);
  }
  *run_before = 0.f;
  return __shfl(item0, 0);
}

// The same search when lane l holds NE consecutive items of each of NG groups, the
// groups following each other: item = first + g * gstride + l * NE + e (gstride =
// 64 * NE).  Items past the end must carry weight 0.  Each load instruction of such a
// layout reads one contiguous run (lane-interleaved), unlike a per-lane contiguous one.
template <int NG, int NE>
__device__ int wave_find_grouped(const float (&w)[NG][NE], int first, float base, float target, float *run_before) {
  const int lane = threadIdx.x & 63;
  float sg[NG], inc[NG], gt[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) x += w[g][e];
    sg[g] = x;
    inc[g] = wave_incl_scan(x);
    gt[g] = __shfl(inc[g], 63);
  }
  // the group holding the draw (uniform over the wave)
  float run = base, gbase = 0.f, lbase = 0.f;
  int gs = -1, gl = -1;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (gt[g] > 0.f) {
      if (gs < 0 && run + gt[g] > target) {
        gs = g;
        gbase = run;
      }
      gl = g;
      lbase = run;
    }
    run += gt[g];
  }
  float tgt = target;
  if (gs < 0) {
    if (gl < 0) {
      *run_before = base;
      return first;
    }
    gs = gl;  // rounding left the target beyond the end: the last item of positive weight
    gbase = lbase;
    tgt = INFINITY;
  }
  float ws[NE], ss = 0.f, is = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) ws[e] = 0.f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g == gs) {
#pragma unroll
      for (int e = 0; e < NE; ++e) ws[e] = w[g][e];
      ss = sg[g];
      is = inc[g];
    }
  }
  return wave_find(ws, NE, first + gs * 64 * NE + lane * NE, gbase, is, ss, tgt, run_before);
}

constexpr int T2_CG = 4;     // groups of 64 chunk sums in a draw (C <= 256)
constexpr int T2_NT2 = 512;  // threads reading the chosen chunk in a draw, 4 tokens each (chunk <= 2048)

// The draw of one token by inverse CDF.  csums holds, per chunk of `chunk` tokens, the sum
// of max(0, p - q) and the sum of p over the chunk (q from z2; without z2, or when all of
// max(0, p - q) is zero, the draw is from p).  The chunk holding u * total comes from the
// chunk sums (every wave finds it), the token from that chunk's logits: thread t holds
// tokens 4t .. 4t+3 of the chunk and a block scan locates the draw.  Called by all T2_NT2
// threads of the block; every thread gets the token.
template <bool VEC>
__device__ int pick_token(const float *z1, const float *z2, float lse1, float lse2, float u, const float *csums, int C,
                          int chunk, int V, float invT, float *s_wt, int *s_v) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  float wr[T2_CG][1], wp[T2_CG][1];
#pragma unroll
  for (int g = 0; g < T2_CG; ++g) {
    const int c = 64 * g + lane;
    float2 v = make_float2(0.f, 0.f);
    if (c < C) v = *reinterpret_cast<const float2 *>(csums + 2 * (long)c);
    wr[g][0] = v.x;
    wp[g][0] = v.y;
  }
  float lr = 0.f, lp = 0.f;
#pragma unroll
  for (int g = 0; g < T2_CG; ++g) {
    lr += wr[g][0];
    lp += wp[g][0];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lr += __shfl_xor(lr, off);
    lp += __shfl_xor(lp, off);
  }
  const bool resid = z2 != nullptr && lr > 0.f;
  const float target = u * (resid ? lr : lp);
  float base;
  const int pick = resid ? wave_find_grouped(wr, 0, 0.f, target, &base) : wave_find_grouped(wp, 0, 0.f, target, &base);
  const float *zq = resid ? z2 : nullptr;
  const int v0 = pick * chunk, v1 = min(V, v0 + chunk);
  const int vt = v0 + 4 * t;
  float zt[4], zd[4];
  if constexpr (VEC) {
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const f32x4 xv = vt < v1 ? *reinterpret_cast<const f32x4 *>(z1 + vt) : zero4;
    const f32x4 yv = (zq && vt < v1) ? *reinterpret_cast<const f32x4 *>(zq + vt) : zero4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      zt[e] = xv[e];
      zd[e] = yv[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      zt[e] = vt + e < v1 ? z1[vt + e] : 0.f;
      zd[e] = (zq && vt + e < v1) ? zq[vt + e] : 0.f;
    }
  }
  float w4[4];
  float mine = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float xw = 0.f;
    if (vt + e < v1) {
      const float p = __expf(zt[e] * invT - lse1);
      xw = resid ? fmaxf(p - __expf(zd[e] * invT - lse2), 0.f) : p;
    }
    w4[e] = xw;
    mine += xw;
  }
  const float incl = wave_incl_scan(mine);
  if (lane == 63) s_wt[wave] = incl;
  __syncthreads();
  // the wave holding the draw (same decision in every wave)
  float run = base, hbase = 0.f, lbase = 0.f;
  int hw = -1, lw = -1;
#pragma unroll
  for (int w = 0; w < T2_NT2 / 64; ++w) {
    const float x = s_wt[w];
    if (x > 0.f) {
      if (hw < 0 && run + x > target) {
        hw = w;
        hbase = run;
      }
      lw = w;
      lbase = run;
    }
    run += x;
  }
  float tgt = target;
  if (hw < 0) {  // rounding left the target beyond the end: the last token of positive weight
    hw = lw;
    hbase = lbase;
    tgt = INFINITY;
  }
  if (hw < 0) {
    if (t == 0) *s_v = min(max(v0, 0), V - 1);
  } else if (wave == hw) {
    float dummy;
    const int v = wave_find(w4, 4, vt, hbase, incl, mine, tgt, &dummy);
    if (lane == 0) *s_v = min(max(v, 0), V - 1);
  }
  __syncthreads();
  return *s_v;
}

// Merge two rows' statistic partials with one wave, the loads of both rows issued
// together (BATCH per lane and row at a time); p1 may be null.  Same order of merges as
// wave_merge_row, so the same results.  after_issue() runs once every load of the first
// batch has been issued (a caller's own loads go there, behind the partials).
template <int BATCH, typename F>
__device__ void wave_merge_rows2(const StatPart *p0, const StatPart *p1, int nslots, float invT, StatPart &o0,
                                 StatPart &o1, F after_issue) {
  const int lane = threadIdx.x & 63;
  StatPart s0 = stat_empty(), s1 = stat_empty();
  for (int i0 = 0; i0 < nslots; i0 += 64 * BATCH) {
    StatPart q0[BATCH], q1[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int i = i0 + 64 * k + lane;
      q0[k] = i < nslots ? p0[i] : stat_empty();
      q1[k] = (p1 && i < nslots) ? p1[i] : stat_empty();
    }
    if (i0 == 0) after_issue();
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      s0 = stat_merge(s0, q0[k], invT, true);
      if (p1) s1 = stat_merge(s1, q1[k], invT, true);
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    s0 = stat_merge(s0, stat_shfl_xor(s0, off), invT, true);
    if (p1) s1 = stat_merge(s1, stat_shfl_xor(s1, off), invT, true);
  }
  o0 = s0;
  o1 = s1;
}

// ---- small-batch tail (B * (K+1) <= 32), two kernels, no inter-block signalling.
// tail_a, blocks (pair of sampling chunks, request): every block merges its request's row
// statistics (one wave per pair of rows; the draft ids and coins are loaded first, the
// logits at the draft ids right behind the statistic partials), decides acceptance left
// to right (Wildberries page, "A bit of theory", Statement 1: u < p(x)/q(x)), and
// sums the sampling weights of the draw at the first rejection A over its two chunks:
// max(0, p - q) and p from target row A and draft row A (p alone for the bonus row
// A = K_b).  So only the accepted candidate's two rows are read.  The request's first
// block also writes A, the accepted length, the row diagnostics and the device status.
// tail_b, one block per request: the draw (pick_token) with the request's final coin and
// the emitted tokens; its block 0 writes tau and the counters.
constexpr int TA_NT = 1024;  // tail_a: 512 threads per chunk, 4 tokens each

template <bool VEC>
__global__ __launch_bounds__(TA_NT) void k_tail_a(const AcceptArgs a, int chunk, int C, float *sums, float *req) {
  __shared__ float s_lse_t[64], s_lse_d[64];
  __shared__ int s_rowbad[128];
  __shared__ int s_A;
  __shared__ float s_red[TA_NT / 64][2];
  const int Kmax = a.K;
  const int b = blockIdx.y, cb = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  constexpr int NW = TA_NT / 64;
  const int Kb = a.verify_len ? a.verify_len[b] : Kmax;
  const long trow0 = a.row_off ? a.row_off[b] : (long)b * (Kmax + 1);
  const long drow0 = (long)b * Kmax;
  const float invT = a.invT;
  const bool lead = cb == 0;  // the request's first block writes its results
  // wave 0: the inputs of the first 64 acceptance decisions.  The draft ids and coins
  // are loaded first; the logits at the ids are loaded once the ids are in, after this
  // wave's statistic partials have been requested (so its merges do not wait for them).
  int x0 = 0;
  float u0 = 0.f, zt0 = 0.f, zd0 = 0.f;
  if (wave == 0 && lane < Kb) {
    x0 = a.draft[drow0 + lane];
    u0 = a.u[(long)b * (Kmax + 1) + lane];
  }
  auto load_at_drafts = [&]() {
    if (wave == 0 && lane < Kb && x0 >= 0 && x0 < a.V) {
      zt0 = a.logits_t[(trow0 + lane) * (long)a.V + x0];
      zd0 = a.logits_d[(drow0 + lane) * (long)a.V + x0];
    }
  };
  // row statistics: rows r = 0..Kb are target rows, r = Kb+1..2Kb draft rows 0..Kb-1
  const int nrows = 2 * Kb + 1;
  auto rowp = [&](int r) -> const StatPart * {
    if (r >= nrows) return nullptr;
    return r <= Kb ? a.parts_t + (trow0 + r) * a.nslots_t : a.parts_d + (drow0 + r - Kb - 1) * a.nslots_d;
  };
  auto finish_row = [&](int r, const StatPart &st) {
    const bool is_t = r <= Kb;
    const int j = is_t ? r : r - Kb - 1;
    const float lse = st.b1 * invT + __logf(st.s);
    if (lane == 0) {
      if (is_t) s_lse_t[j] = lse; else s_lse_d[j] = lse;
      s_rowbad[r] = isfinite(lse) ? 0 : 1;
      if (lead && a.diag) {
        const long drow = is_t ? (long)b * (Kmax + 1) + j : (long)a.B * (Kmax + 1) + drow0 + j;
        float *dg = a.diag + drow * SV_DIAG_COLS;
        dg[0] = lse; dg[1] = (float)st.i1; dg[2] = st.b1 - st.b2; dg[3] = st.b1;
        dg[4] = NAN; dg[5] = NAN; dg[6] = is_t ? NAN : 1.f / st.s; dg[7] = 0.f;
      }
    }
  };
  bool drafts_loaded = false;
  for (int r0 = wave; r0 < nrows; r0 += 2 * NW) {
    const int r1 = r0 + NW;
    if (a.nslots_t == a.nslots_d || (r0 <= Kb) == (r1 <= Kb)) {
      const int ns = r0 <= Kb ? a.nslots_t : a.nslots_d;
      StatPart s0, s1;
      wave_merge_rows2<4>(rowp(r0), rowp(r1), ns, invT, s0, s1, [&]() {
        if (!drafts_loaded) load_at_drafts();
        drafts_loaded = true;
      });
      finish_row(r0, s0);
      if (r1 < nrows) finish_row(r1, s1);
    } else {
      if (!drafts_loaded) load_at_drafts();
      drafts_loaded = true;
      finish_row(r0, wave_merge_row<8>(rowp(r0), r0 <= Kb ? a.nslots_t : a.nslots_d, invT, true));
      if (r1 < nrows) finish_row(r1, wave_merge_row<8>(rowp(r1), r1 <= Kb ? a.nslots_t : a.nslots_d, invT, true));
    }
  }
  if (!drafts_loaded) load_at_drafts();  // a wave with no rows (only when Kb is small)
  __syncthreads();
  // acceptance, left to right: lane j of wave 0 handles draft position j+1
  if (wave == 0) {
    bool ok = true, rej = false;
    int A = 0;
    for (int base = 0; base < Kb; base += 64) {
      const int j = base + lane;
      bool acc = false, bad_tok = false;
      if (j < Kb) {
        const int x = base == 0 ? x0 : a.draft[drow0 + j];
        if (x < 0 || x >= a.V) {
          bad_tok = true;
        } else {
          const float zt = base == 0 ? zt0 : a.logits_t[(trow0 + j) * (long)a.V + x];
          const float zd = base == 0 ? zd0 : a.logits_d[(drow0 + j) * (long)a.V + x];
          const float lpt = zt * invT - s_lse_t[j];
          const float lqd = zd * invT - s_lse_d[j];
          const float ratio = __expf(lpt - lqd);
          const float u = base == 0 ? u0 : a.u[(long)b * (Kmax + 1) + j];
          acc = u < ratio;
          if (lead && a.diag) {
            float *dt = a.diag + ((long)b * (Kmax + 1) + j) * SV_DIAG_COLS;
            dt[4] = zt; dt[5] = __expf(lpt); dt[6] = ratio;
            float *dd = a.diag + ((long)a.B * (Kmax + 1) + drow0 + j) * SV_DIAG_COLS;
            dd[4] = zd; dd[5] = __expf(lqd);
          }
        }
      }
      if (__any(bad_tok)) ok = false;
      if (!rej) {
        const unsigned long long live = (Kb - base >= 64) ? ~0ull : ((1ull << (Kb - base)) - 1ull);
        const unsigned long long rejm = __ballot(!acc) & live;
        if (rejm) {
          A = base + __ffsll((long long)rejm) - 1;
          rej = true;
        } else {
          A = min(Kb, base + 64);
        }
      }
    }
    int rb = 0;
    for (int r = lane; r < nrows; r += 64) rb |= s_rowbad[r];
    const bool nonfinite = __any(rb != 0);
    if (lane == 0) {
      const bool good = ok && !nonfinite;
      s_A = good ? A : -1;
      if (lead) {
        if (!ok) set_status(a.dev_status, SV_DEV_BAD_TOKEN);
        if (nonfinite) set_status(a.dev_status, SV_DEV_NONFINITE);
        a.accepted_len[b] = good ? A : -1;
      }
    }
  }
  __syncthreads();
  const int A = s_A;
  if (A < 0) {
    if (lead && t == 0) req[3 * b] = __int_as_float(-1);
    return;
  }
  // sampling weights of the draw at A over this block's chunks 2 cb and 2 cb + 1
  const bool resid = A < Kb;
  const float lse1 = s_lse_t[A], lse2 = resid ? s_lse_d[A] : 0.f;
  const float *z1 = a.logits_t + (trow0 + A) * (long)a.V;
  const float *z2 = resid ? a.logits_d + (drow0 + A) * (long)a.V : nullptr;
  const int c = 2 * cb + (t >> 9);
  const int v0 = c * chunk, v1 = min(a.V, v0 + chunk);
  const int vt = v0 + 4 * (t & 511);
  float zt[4], zd[4];
  if constexpr (VEC) {
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const f32x4 xv = vt < v1 ? *reinterpret_cast<const f32x4 *>(z1 + vt) : zero4;
    const f32x4 yv = (z2 && vt < v1) ? *reinterpret_cast<const f32x4 *>(z2 + vt) : zero4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      zt[e] = xv[e];
      zd[e] = yv[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      zt[e] = vt + e < v1 ? z1[vt + e] : 0.f;
      zd[e] = (z2 && vt + e < v1) ? z2[vt + e] : 0.f;
    }
  }
  float sr = 0.f, sp = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (vt + e < v1) {
      const float p = __expf(zt[e] * invT - lse1);
      sp += p;
      if (z2) sr += fmaxf(p - __expf(zd[e] * invT - lse2), 0.f);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sr += __shfl_xor(sr, off);
    sp += __shfl_xor(sp, off);
  }
  if (lane == 0) {
    s_red[wave][0] = sr;
    s_red[wave][1] = sp;
  }
  __syncthreads();
  if (t < 4) {
    const int h = t >> 1, k = t & 1;  // chunk 2 cb + h: waves 8 h .. 8 h + 7, in order
    float tot = 0.f;
    for (int w = 8 * h; w < 8 * h + 8; ++w) tot += s_red[w][k];
    const int cc = 2 * cb + h;
    if (cc < C) sums[((long)b * C + cc) * 2 + k] = tot;
  }
  if (lead && t == 0) {
    req[3 * b] = __int_as_float(A);
    req[3 * b + 1] = lse1;
    req[3 * b + 2] = lse2;
  }
}

template <bool VEC>
__global__ __launch_bounds__(T2_NT2) void k_tail_b(const AcceptArgs a, int chunk, int C, const float *sums,
                                                   const float *req, FinalizeArgs fin) {
  __shared__ float s_wt[T2_NT2 / 64];
  __shared__ int s_v;
  const int Kmax = a.K, b = blockIdx.x, t = threadIdx.x;
  const int A = __float_as_int(req[3 * b]);
  const int Kb = a.verify_len ? a.verify_len[b] : Kmax;
  const long trow0 = a.row_off ? a.row_off[b] : (long)b * (Kmax + 1);
  const long drow0 = (long)b * Kmax;
  int v = -1;
  if (A >= 0) {
    const float *z1 = a.logits_t + (trow0 + A) * (long)a.V;
    const float *z2 = A < Kb ? a.logits_d + (drow0 + A) * (long)a.V : nullptr;
    v = pick_token<VEC>(z1, z2, req[3 * b + 1], req[3 * b + 2], a.u[(long)b * (Kmax + 1) + Kmax],
                        sums + (long)b * C * 2, C, chunk, a.V, a.invT, s_wt, &s_v);
  }
  for (int jj = t; jj <= Kmax; jj += blockDim.x) {
    int e = -1;
    if (A >= 0) {
      if (jj < A) e = a.draft[drow0 + jj];
      if (jj == A) e = v;
    }
    a.emitted[(long)b * (Kmax + 1) + jj] = e;
  }
  if (b == 0 && fin.acc) finalize_block(fin);
}

// ---- inverse-CDF sampling of one token per job (larger batches, drafter step), two
// kernels with no inter-block signalling: sample_sums sums the weights of every job over
// SUBS chunks per block; sample_pick (one block per job) finds the chunk from those sums
// and the token inside it (pick_token); its block 0 also writes the call-wide
// bookkeeping (the accepted lengths are final before the draw).  The weight of token v
// is max(0, p_v - q_v) (p_v if the job has no second row or all of those are zero),
// recomputed from the fp32 logits in ascending token order.
template <bool VEC>
__global__ __launch_bounds__(NT) void k_sample_sums(const SampleJob *jobs, int V, int chunk, int C, float invT,
                                                    float *sums) {
  __shared__ float red[NT / 64][2 * SUBS];
  const int job = blockIdx.y, cb = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const SampleJob jb = jobs[job];
  if (jb.out_index < 0) return;
  const float *z1 = jb.z1, *z2 = jb.z2;
  auto tok = [&](int q, int i) {
    const int v0 = (cb * SUBS + q) * chunk;
    return VEC ? v0 + (i >> 2) * (4 * NT) + 4 * t + (i & 3) : v0 + t + i * NT;
  };
  float zt[SUBS][PER], zd[SUBS][PER];
#pragma unroll
  for (int q = 0; q < SUBS; ++q) {
    const int v1 = min(V, (cb * SUBS + q) * chunk + chunk);
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < PER; i += 4) {
        const int v = tok(q, i);
        const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
        const f32x4 xv = v < v1 ? *reinterpret_cast<const f32x4 *>(z1 + v) : zero4;
        const f32x4 yv = (z2 && v < v1) ? *reinterpret_cast<const f32x4 *>(z2 + v) : zero4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          zt[q][i + e] = xv[e];
          zd[q][i + e] = yv[e];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int v = tok(q, i);
        zt[q][i] = v < v1 ? z1[v] : 0.f;
        zd[q][i] = (z2 && v < v1) ? z2[v] : 0.f;
      }
    }
  }
  float part[2 * SUBS];
#pragma unroll
  for (int q = 0; q < SUBS; ++q) {
    const int v1 = min(V, (cb * SUBS + q) * chunk + chunk);
    float sr = 0.f, sp = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (tok(q, i) < v1) {
        const float p = __expf(zt[q][i] * invT - jb.lse1);
        sp += p;
        if (z2) sr += fmaxf(p - __expf(zd[q][i] * invT - jb.lse2), 0.f);
      }
    }
    part[2 * q] = sr;
    part[2 * q + 1] = sp;
  }
#pragma unroll
  for (int k = 0; k < 2 * SUBS; ++k) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part[k] += __shfl_xor(part[k], off);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 2 * SUBS; ++k) red[wave][k] = part[k];
  }
  __syncthreads();
  if (t < 2 * SUBS) {
    const int c = cb * SUBS + (t >> 1);
    float tot = 0.f;
    for (int w = 0; w < NT / 64; ++w) tot += red[w][t];
    if (c < C) sums[((long)job * C + c) * 2 + (t & 1)] = tot;
  }
}

template <bool VEC>
__global__ __launch_bounds__(T2_NT2) void k_sample_pick(const SampleJob *jobs, int V, int chunk, int C, float invT,
                                                        const float *sums, int32_t *out, FinalizeArgs fin) {
  __shared__ float s_wt[T2_NT2 / 64];
  __shared__ int s_v;
  const int job = blockIdx.x;
  const SampleJob jb = jobs[job];
  if (jb.out_index >= 0) {
    const int v = pick_token<VEC>(jb.z1, jb.z2, jb.lse1, jb.lse2, jb.u, sums + (long)job * C * 2, C, chunk, V, invT,
                                  s_wt, &s_v);
    if (threadIdx.x == 0) out[jb.out_index] = v;
  }
  if (job == 0 && fin.acc) finalize_block(fin);
}

// Confidence of each draft row: conf = max_v q(v) = 1 / sum_v exp((z_v - max z)/T).  One wave per row.
__global__ __launch_bounds__(NT) void k_row_conf(const StatPart *parts, int nslots, int rows, float invT,
                                                 float *conf, int32_t *dev_status, float *diag, long diag_row0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * (NT / 64) + wave;
  if (r >= rows) return;
  const StatPart st = wave_merge_row<12>(parts + (long)r * nslots, nslots, invT, true);
  if (lane == 0) {
    conf[r] = 1.f / st.s;
    if (!isfinite(st.b1) || !(st.s >= 1.f)) set_status(dev_status, SV_DEV_NONFINITE);
    if (diag) {
      float *dg = diag + (diag_row0 + r) * SV_DIAG_COLS;
      dg[0] = st.b1 * invT + __logf(st.s); dg[1] = (float)st.i1; dg[2] = st.b1 - st.b2; dg[3] = st.b1;
      dg[4] = NAN; dg[5] = NAN; dg[6] = 1.f / st.s; dg[7] = 0.f;
    }
  }
}

// ---- confidence schedule (single block).
// Exclusive prefix sum of v over the block in thread order (blockDim.x <= 1024); *total
// gets the block total.  buf needs 16 ints.  Every thread must call it.
__device__ int block_excl_scan_int(int v, int *buf, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int bw = buf[w];
    if (w < wave) base += bw;
    tot += bw;
  }
  *total = tot;
  return base + x - v;
}

// The verify length of every request (one block of 1024 threads).  Survival s_b(k) is
// the running product of the draft confidences; entries with s >= threshold are
// eligible (a prefix of each request).  When the eligible entries exceed the budget
// beyond the B target rows (R), the R entries with the largest key floor(1024 s) are
// kept, ties in (request, position) order: the cut key comes from a suffix scan of the
// key histogram, the rank of each entry at the cut key from a prefix scan.  Because keys
// do not increase along a request, the kept entries are a prefix of each request.
__global__ __launch_bounds__(1024) void k_schedule(const ScheduleArgs a) {
  extern __shared__ int smi[];
  const int B = a.B, Km = a.Kmax, n = B * Km;
  int *keys = smi;          // [n]   confidences (as float bits), then keys: -1 if not eligible
  int *hist = smi + n;      // [1025]
  int *kb = hist + 1025;    // [B]
  __shared__ int s_buf[16];
  __shared__ int s_nelig, s_cut, s_take, s_S1;
  const int tid = threadIdx.x, nt = blockDim.x;
  if (a.status_reset && tid == 0) *a.status_reset = 0;
  for (int i = tid; i < n; i += nt) keys[i] = __float_as_int(a.conf[i]);
  for (int i = tid; i < 1025; i += nt) hist[i] = 0;
  if (tid == 0) {
    s_nelig = 0;
    s_cut = -2;
  }
  __syncthreads();
  // survival products per request (fp32, ascending k) and keys
  for (int b = tid; b < B; b += nt) {
    float sv = 1.f;
    int lead = 0;
    bool alive = true;
    for (int k = 0; k < Km; ++k) {
      sv *= __int_as_float(keys[b * Km + k]);
      const bool el = alive && (sv >= a.threshold);
      alive = el;
      keys[b * Km + k] = el ? (int)floorf(1024.f * sv) : -1;
      if (el) ++lead;
    }
    kb[b] = lead;
    atomicAdd(&s_nelig, lead);
  }
  __syncthreads();
  const int R = a.budget - B;  // positions that may be added beyond the B target rows
  if (s_nelig > R) {           // block-uniform
    for (int i = tid; i < n; i += nt)
      if (keys[i] >= 0) atomicAdd(&hist[min(keys[i], 1024)], 1);
    for (int b = tid; b < B; b += nt) kb[b] = 0;
    __syncthreads();
    // S(c) = number of eligible keys >= c; thread t covers c = 1024 - t (c >= 1)
    {
      const int c = 1024 - tid;
      const int h = (tid < 1024 && c >= 1) ? hist[c] : 0;
      int tot;
      const int excl = block_excl_scan_int(h, s_buf, &tot);
      const int incl = excl + h;  // S(c); excl = S(c + 1)
      if (tid < 1024 && c >= 1 && incl >= R && excl < R) {
        s_cut = c;
        s_take = R - excl;
      }
      if (c == 1) s_S1 = incl;
    }
    __syncthreads();
    if (tid == 0 && s_cut == -2) {
      if (R <= 0) {  // nothing beyond the target rows: the cut sits above every key
        s_cut = 1024;
        s_take = 0;
      } else {       // S(1) < R <= S(0)
        s_cut = 0;
        s_take = R - s_S1;
      }
    }
    __syncthreads();
    const int cut = s_cut, take = s_take;
    // rank of each entry at the cut key in (request, position) order, 1024 entries a pass
    int carry = 0;
    for (int i0 = 0; i0 < n; i0 += nt) {
      const int i = i0 + tid;
      const int key = i < n ? keys[i] : -1;
      int tot;
      const int rank = carry + block_excl_scan_int(key == cut ? 1 : 0, s_buf, &tot);
      if (i < n && (key > cut || (key == cut && rank < take))) atomicAdd(&kb[i / Km], 1);
      carry += tot;
    }
    __syncthreads();
  }
  // offsets (exclusive scan of k_b + 1), the packed row map and the verify lengths
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += nt) {
    const int b = b0 + tid;
    const int len = b < B ? kb[b] + 1 : 0;
    int tot;
    const int off = carry + block_excl_scan_int(len, s_buf, &tot);
    if (b < B) {
      a.row_off[b] = off;
      for (int j = 0; j < len; ++j) a.row_map[off + j] = b * (Km + 1) + j;
      a.verify_len[b] = len - 1;
      if (a.verify_len_out) a.verify_len_out[b] = len - 1;
    }
    carry += tot;
  }
  if (tid == 0) {
    a.row_off[B] = carry;
    *a.m_total = carry;
  }
}

__global__ void k_gather_rows(const uint16_t *src, uint16_t *dst, const int32_t *row_map, const int32_t *m_total,
                              int d) {
  const int r = blockIdx.x;
  if (r >= *m_total) return;
  const long s = (long)row_map[r] * d, t = (long)r * d;
  for (int i = threadIdx.x * 8; i < d; i += blockDim.x * 8)
    *reinterpret_cast<u32x4 *>(dst + t + i) = *reinterpret_cast<const u32x4 *>(src + s + i);
}

__global__ void k_scatter_f32(const float *packed, float *dst, const int32_t *row_map, const int32_t *m_total,
                              int V) {
  const int r = blockIdx.x;
  if (r >= *m_total) return;
  const long s = (long)r * V, t = (long)row_map[r] * V;
  for (int i = threadIdx.x; i < V; i += blockDim.x) dst[t + i] = packed[s + i];
}

__global__ void k_scatter_u16(const uint16_t *packed, uint16_t *dst, const int32_t *row_map,
                              const int32_t *m_total, int d) {
  const int r = blockIdx.x;
  if (r >= *m_total) return;
  const long s = (long)r * d, t = (long)row_map[r] * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) dst[t + i] = packed[s + i];
}

// Propose mode: per draft row, argmax (T == 0) or a sampling job from q.
__global__ __launch_bounds__(NT) void k_propose_finish(const StatPart *parts, int nslots, int rows, float invT,
                                                       float T, const float *logits, int V, const float *coins,
                                                       SampleJob *jobs, int32_t *draft_out, float *conf_out,
                                                       int32_t *dev_status, int32_t *job_cnt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.x * (NT / 64) + wave;
  if (r >= rows) return;
  const bool samp = T > 0.f;
  const StatPart st = wave_merge_row<12>(parts + (long)r * nslots, nslots, samp ? invT : 1.f, samp);
  if (lane != 0) return;
  job_cnt[r] = 0;
  const float lse = st.b1 * invT + __logf(st.s);
  const bool fin = isfinite(st.b1) && (!samp || isfinite(lse));
  if (!fin) set_status(dev_status, SV_DEV_NONFINITE);
  if (!samp) {
    draft_out[r] = fin ? st.i1 : -1;
    if (conf_out) conf_out[r] = 1.f;
    return;
  }
  if (conf_out) conf_out[r] = 1.f / st.s;
  SampleJob jb;
  jb.z1 = logits + (long)r * V;
  jb.z2 = nullptr;
  jb.lse1 = lse;
  jb.lse2 = 0.f;
  jb.u = coins[r];
  jb.out_index = fin ? r : -1;
  jobs[r] = jb;
  if (!fin) draft_out[r] = -1;
}


// ---- tree verification: one block of TNT threads per request.  The tree (at most 64
// nodes) and every row's statistics sit in LDS; the walk is block-uniform: every thread
// takes the same decisions from the same values.  After j failed candidates at node u
// the residual is max(0, p_u - c q_u) / Z (c_0 = 0, Z_0 = 1, c_{j+1} = c_j + Z_j,
// Z_{j+1} = sum_v max(0, p_u(v) - c_{j+1} q_u(v))): the normalised max(0, r - q_u) of
// the previous residual r written in closed form, so each failed candidate costs one
// pass over the two rows.  The pass keeps the sums of 64-token chunks in LDS, from
// which the final inverse-CDF draw finds its chunk without another pass.
constexpr int TNT = 1024;
constexpr int TCH = 256;                   // tokens per chunk: 4 per lane of a wave
constexpr int TMAXCH = (1 << 19) / TCH;    // chunks of the largest vocabulary
constexpr int TU = 4;                      // chunks per wave whose loads are in flight together

struct TreeRows {
  const float *zt, *zd;  // target / draft logit rows of the current node (zd null: r = p)
  float lt, ld, invT, cc;
};

__device__ __forceinline__ float tree_w1(const TreeRows &r, float zt, float zd) {
  const float p = __expf(zt * r.invT - r.lt);
  if (!r.zd) return p;
  return fmaxf(p - r.cc * __expf(zd * r.invT - r.ld), 0.f);
}

// The residual weights of tokens [v0, v0 + 4) (zero past V); 16-byte loads when VEC.
template <bool VEC>
__device__ __forceinline__ void tree_w4(const TreeRows &r, int v0, int V, float w[4]) {
  if (VEC && v0 + 3 < V) {
    const f32x4 t = *reinterpret_cast<const f32x4 *>(r.zt + v0);
    f32x4 d = t;
    if (r.zd) d = *reinterpret_cast<const f32x4 *>(r.zd + v0);
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = tree_w1(r, t[k], d[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int v = v0 + k;
      w[k] = v < V ? tree_w1(r, r.zt[v], r.zd ? r.zd[v] : 0.f) : 0.f;
    }
  }
}

// Sums of the residual weights per 256-token chunk into csum, and their total (fixed
// order).  Each wave takes chunks wave, wave + 16, ...; TU of them are loaded at once.
template <bool VEC>
__device__ float tree_sums(const TreeRows &r, int V, float *csum, float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = TNT / 64;
  const int nch = (V + TCH - 1) / TCH;
  for (int ch0 = wave; ch0 < nch; ch0 += NW * TU) {
    float w[TU][4];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int ch = ch0 + u * NW;
      if (ch < nch) tree_w4<VEC>(r, ch * TCH + 4 * lane, V, w[u]);
      else w[u][0] = w[u][1] = w[u][2] = w[u][3] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      float t = (w[u][0] + w[u][1]) + (w[u][2] + w[u][3]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
      const int ch = ch0 + u * NW;
      if (lane == 0 && ch < nch) csum[ch] = t;
    }
  }
  __syncthreads();
  float s = 0.f;
  for (int i = threadIdx.x; i < nch; i += TNT) s += csum[i];
  return block_sum(s, red);
}

// Inverse-CDF draw over ascending ids: the first v whose running weight exceeds
// coin * total; with rounding past the end, the last token of positive weight.
template <bool VEC>
__device__ int tree_draw(const TreeRows &r, int V, float total, float coin, const float *csum, float *scan,
                         int *redi, float *sbase) {
  const int nch = (V + TCH - 1) / TCH;
  const int per = (nch + TNT - 1) / TNT;
  const float target = coin * total;
  float loc = 0.f;
  for (int i = 0; i < per; ++i) {
    const int ch = threadIdx.x * per + i;
    if (ch < nch) loc += csum[ch];
  }
  const float incl = block_incl_scan(loc, scan);
  int found = 0x7fffffff, last = -1;
  float run = incl - loc;
  for (int i = 0; i < per; ++i) {
    const int ch = threadIdx.x * per + i;
    if (ch >= nch) break;
    if (csum[ch] > 0.f) last = ch;
    if (found == 0x7fffffff && run <= target && run + csum[ch] > target) {
      found = ch;
      *sbase = run;  // one writer: the chunk whose running sum crosses the target
    }
    run += csum[ch];
  }
  const int fch = block_min_int(found, redi);
  int lch = fch;
  float base = 0.f;
  if (fch == 0x7fffffff) {  // rounding: fall back to the last chunk with weight
    lch = -block_min_int(-last, redi);
    if (lch < 0) return 0;
  } else {
    __syncthreads();
    base = *sbase;
  }
  __shared__ int stok;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float w[4];
    tree_w4<VEC>(r, lch * TCH + 4 * lane, V, w);
    const float own = (w[0] + w[1]) + (w[2] + w[3]);
    float c = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float x = __shfl_up(c, off);
      if (lane >= off) c += x;
    }
    float run_l = base + (c - own);  // before this lane's 4 tokens
    int hitk = -1, lastk = -1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (w[k] > 0.f) lastk = k;
      if (hitk < 0 && fch != 0x7fffffff && run_l + w[k] > target) hitk = k;
      run_l += w[k];
    }
    const unsigned long long hit = __ballot(hitk >= 0);
    const unsigned long long pos = __ballot(lastk >= 0);
    const int hl = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : 0);
    const int hk = __shfl(hit ? hitk : lastk, hl);
    if (lane == 0) stok = lch * TCH + 4 * hl + (hk < 0 ? 0 : hk);
  }
  __syncthreads();
  return stok;
}

template <bool VEC>
__global__ __launch_bounds__(TNT) void k_tree(const TreeArgs a) {
  __shared__ float s_lse_t[64], s_lse_d[64];
  __shared__ int s_amax[64], s_par[64], s_tok[64], s_path[64];
  __shared__ float csum[TMAXCH];
  __shared__ float red[TNT / 64], scan[TNT / 64], sbase;
  __shared__ int redi[TNT / 64], flag, s_err;
  const int b = blockIdx.x, K = a.K, N = K + 1, V = a.V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long trow0 = (long)b * N, drow0 = (long)b * K;
  const bool samp = !a.greedy;
  if (tid == 0) s_err = 0;
  if (tid < K) {
    s_par[tid + 1] = a.parent[drow0 + tid];
    s_tok[tid + 1] = a.tokens[drow0 + tid];
  }
  __syncthreads();
  if (tid < K) {
    const int par = s_par[tid + 1], tok = s_tok[tid + 1];
    if (par < 0 || par > tid) atomicOr(&s_err, 1);
    if (tok < 0 || tok >= V) atomicOr(&s_err, 2);
  }
  const int nrows = N + (samp ? K : 0);
  for (int r = wave; r < nrows; r += TNT / 64) {
    const bool tgt = r < N;
    const int j = tgt ? r : r - N;
    const StatPart st = tgt ? wave_merge_row(a.parts_t + (trow0 + j) * a.nslots_t, a.nslots_t, a.invT,
                                             samp || a.diag)
                            : wave_merge_row(a.parts_d + (drow0 + j) * a.nslots_d, a.nslots_d, a.invT, true);
    if (lane == 0) {
      const float lse = st.b1 * a.invT + __logf(st.s);
      if (tgt) { s_amax[j] = st.i1; s_lse_t[j] = lse; } else { s_lse_d[j] = lse; }
      if (!isfinite(st.b1) || (samp && !isfinite(lse))) atomicOr(&s_err, 4);
      if (a.diag) {
        float *dg = a.diag + (tgt ? trow0 + j : (long)a.B * N + drow0 + j) * SV_DIAG_COLS;
        dg[0] = lse; dg[1] = (float)st.i1; dg[2] = st.b1 - st.b2; dg[3] = st.b1;
        dg[4] = NAN; dg[5] = NAN; dg[6] = NAN; dg[7] = 0.f;
      }
    }
  }
  __syncthreads();
  const int err = s_err;
  int depth = 0, final_tok = -1;
  if (err == 0) {
    if (tid == 0) s_path[0] = 0;
    int node = 0;
    if (!samp) {
      while (true) {  // uniform: LDS values only
        int nxt = -1;
        for (int c = node + 1; c <= K; ++c)
          if (s_par[c] == node && s_tok[c] == s_amax[node]) { nxt = c; break; }
        if (nxt < 0) break;
        node = nxt;
        ++depth;
        if (tid == 0) s_path[depth] = nxt;
      }
      final_tok = s_amax[node];
    } else {
      const float *ub = a.u + (long)b * N;
      while (true) {
        TreeRows rw{a.logits_t + (trow0 + node) * (long)V, nullptr, s_lse_t[node], 0.f, a.invT, 0.f};
        float Z = 1.f;
        bool sums = false;
        int nxt = -1;
        for (int c = node + 1; c <= K; ++c) {
          if (s_par[c] != node) continue;
          const int x = s_tok[c];
          const float *zd = a.logits_d + (drow0 + node) * (long)V;
          const float px = __expf(rw.zt[x] * a.invT - rw.lt);
          const float qx = __expf(zd[x] * a.invT - s_lse_d[node]);
          const float num = fmaxf(px - rw.cc * qx, 0.f);
          const float ratio = qx > 0.f ? num / (Z * qx) : (num > 0.f ? INFINITY : 0.f);
          if (ub[c - 1] < fminf(1.f, ratio)) { nxt = c; break; }
          rw.zd = zd;
          rw.ld = s_lse_d[node];
          rw.cc += Z;
          Z = tree_sums<VEC>(rw, V, csum, red);
          sums = true;
          if (!(Z > 0.f)) {  // nothing left of the residual: back to p_u
            rw.zd = nullptr;
            rw.cc = 0.f;
            Z = 1.f;
            sums = false;
          }
        }
        if (nxt >= 0) {
          node = nxt;
          ++depth;
          if (tid == 0) s_path[depth] = nxt;
          continue;
        }
        if (!sums) Z = tree_sums<VEC>(rw, V, csum, red);
        final_tok = tree_draw<VEC>(rw, V, Z, ub[K], csum, scan, redi, &sbase);
        break;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (err & 1) set_status(a.dev_status, SV_DEV_BAD_TREE);
    else if (err & 2) set_status(a.dev_status, SV_DEV_BAD_TOKEN);
    else if (err & 4) set_status(a.dev_status, SV_DEV_NONFINITE);
    a.accepted_len[b] = err ? -1 : depth;
  }
  for (int j = tid; j <= K; j += TNT) {
    int e = -1, p = -1;
    if (!err && j <= depth) {
      p = s_path[j];
      e = j < depth ? s_tok[s_path[j + 1]] : final_tok;
    }
    a.emitted[trow0 + j] = e;
    if (a.path) a.path[trow0 + j] = p;
  }
  if (a.fin.acc && arrive_last(a.done_cnt, a.B, &flag)) finalize_block(a.fin);
}


// ---- sampled trees over G blocks per request.  Every block merges the row statistics and
// walks the tree exactly as the others (same values, same order); a residual pass sums one
// slice of the vocabulary per block and publishes the slice total, and the blocks of the
// request meet before reading all totals in a fixed order.  Block 0 draws the final
// token from the chunk sums of the last pass and writes the outputs.

// Arrive at the request's counter and wait until `target` blocks have arrived.  The wait
// is bounded: past `limit` polls it gives up and returns false.  The shared values are
// written and read with device-scope atomics, all stores of a block by the wave that
// arrives; device-scope fences order them against the counter.
__device__ bool tree_meet(int32_t *cnt, int target, int limit) {
  __shared__ int s_ok;
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    atomicAdd(cnt, 1);
    int polls = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target && polls < limit) {
      __builtin_amdgcn_s_sleep(2);
      ++polls;
    }
    __threadfence();
    s_ok = polls < limit;
  }
  __syncthreads();
  return s_ok != 0;
}

// Chunk sums of chunks [c0, c1) into the block's LDS (ls[ch - c0]) and their total
// (fixed order).
template <bool VEC>
__device__ float tree_slice_sums(const TreeRows &r, int V, int c0, int c1, float *ls, float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = TNT / 64;
  float tot = 0.f;
  for (int ch0 = c0 + wave; ch0 < c1; ch0 += NW * TU) {
    float w[TU][4];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int ch = ch0 + u * NW;
      if (ch < c1) tree_w4<VEC>(r, ch * TCH + 4 * lane, V, w[u]);
      else w[u][0] = w[u][1] = w[u][2] = w[u][3] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      float t = (w[u][0] + w[u][1]) + (w[u][2] + w[u][3]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
      const int ch = ch0 + u * NW;
      if (ch < c1) {
        if (lane == 0) ls[ch - c0] = t;
        tot += t;
      }
    }
  }
  return block_sum(lane == 0 ? tot : 0.f, red);
}

template <bool VEC>
__global__ __launch_bounds__(TNT) void k_tree_coop(const TreeArgs a, int G) {
  __shared__ float s_lse_t[64], s_lse_d[64];
  __shared__ int s_par[64], s_tok[64], s_path[64];
  __shared__ float csum[TMAXCH];
  __shared__ float red[TNT / 64], scan[TNT / 64], sbase;
  __shared__ int redi[TNT / 64], flag, s_err;
  const int b = blockIdx.x / G, gi = blockIdx.x % G;
  const int K = a.K, N = K + 1, V = a.V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long trow0 = (long)b * N, drow0 = (long)b * K;
  const int nch = (V + TCH - 1) / TCH;
  const int c0 = (int)((long)gi * nch / G), c1 = (int)((long)(gi + 1) * nch / G);
  float *cs = a.chunk_sums + (long)b * nch;
  float *pt = a.partials + (long)b * 2 * TREE_MAX_BLOCKS;
  if (tid == 0) s_err = 0;
  if (tid < K) {
    s_par[tid + 1] = a.parent[drow0 + tid];
    s_tok[tid + 1] = a.tokens[drow0 + tid];
  }
  __syncthreads();
  if (tid < K) {
    const int par = s_par[tid + 1], tok = s_tok[tid + 1];
    if (par < 0 || par > tid) atomicOr(&s_err, 1);
    if (tok < 0 || tok >= V) atomicOr(&s_err, 2);
  }
  for (int r = wave; r < N + K; r += TNT / 64) {
    const bool tgt = r < N;
    const int j = tgt ? r : r - N;
    const StatPart st = tgt ? wave_merge_row(a.parts_t + (trow0 + j) * a.nslots_t, a.nslots_t, a.invT, true)
                            : wave_merge_row(a.parts_d + (drow0 + j) * a.nslots_d, a.nslots_d, a.invT, true);
    if (lane == 0) {
      const float lse = st.b1 * a.invT + __logf(st.s);
      if (tgt) s_lse_t[j] = lse; else s_lse_d[j] = lse;
      if (!isfinite(st.b1) || !isfinite(lse)) atomicOr(&s_err, 4);
      if (a.diag && gi == 0) {
        float *dg = a.diag + (tgt ? trow0 + j : (long)a.B * N + drow0 + j) * SV_DIAG_COLS;
        dg[0] = lse; dg[1] = (float)st.i1; dg[2] = st.b1 - st.b2; dg[3] = st.b1;
        dg[4] = NAN; dg[5] = NAN; dg[6] = NAN; dg[7] = 0.f;
      }
    }
  }
  __syncthreads();
  int err = s_err;
  int depth = 0, final_tok = -1, pass = 0;
  // one residual pass of the request: every block its slice, then the total of all
  // Wave 0 makes every global store of the pass, so the release in tree_meet (by its
  // lane 0) covers all of them.
  auto coop_sums = [&](const TreeRows &rw) -> float {
    const float loc = tree_slice_sums<VEC>(rw, V, c0, c1, csum, red);
    __syncthreads();
    if (wave == 0) {
      for (int i = lane; i < c1 - c0; i += 64)
        __hip_atomic_store(cs + c0 + i, csum[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0)
        __hip_atomic_store(pt + (pass & 1) * TREE_MAX_BLOCKS + gi, loc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const bool ok = tree_meet(a.meet + b, G * (pass + 1), a.spin_limit);
    float Z = 0.f;
    for (int i = 0; i < G; ++i)
      Z += __hip_atomic_load(pt + (pass & 1) * TREE_MAX_BLOCKS + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ++pass;
    if (!ok) err |= 8;
    return Z;
  };
  if (err == 0) {
    if (tid == 0) s_path[0] = 0;
    int node = 0;
    const float *ub = a.u + (long)b * N;
    while (err == 0) {
      TreeRows rw{a.logits_t + (trow0 + node) * (long)V, nullptr, s_lse_t[node], 0.f, a.invT, 0.f};
      float Z = 1.f;
      bool sums = false;
      int nxt = -1;
      for (int c = node + 1; c <= K && err == 0; ++c) {
        if (s_par[c] != node) continue;
        const int x = s_tok[c];
        const float *zd = a.logits_d + (drow0 + node) * (long)V;
        const float px = __expf(rw.zt[x] * a.invT - rw.lt);
        const float qx = __expf(zd[x] * a.invT - s_lse_d[node]);
        const float num = fmaxf(px - rw.cc * qx, 0.f);
        const float ratio = qx > 0.f ? num / (Z * qx) : (num > 0.f ? INFINITY : 0.f);
        if (ub[c - 1] < fminf(1.f, ratio)) { nxt = c; break; }
        rw.zd = zd;
        rw.ld = s_lse_d[node];
        rw.cc += Z;
        Z = coop_sums(rw);
        sums = true;
        if (!(Z > 0.f)) {
          rw.zd = nullptr;
          rw.cc = 0.f;
          Z = 1.f;
          sums = false;
        }
      }
      if (err) break;
      if (nxt >= 0) {
        node = nxt;
        ++depth;
        if (tid == 0) s_path[depth] = nxt;
        continue;
      }
      if (!sums) Z = coop_sums(rw);
      if (err) break;
      if (gi == 0) {
        for (int i = tid; i < nch; i += TNT) csum[i] = __hip_atomic_load(cs + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        final_tok = tree_draw<VEC>(rw, V, Z, ub[K], csum, scan, redi, &sbase);
      }
      break;
    }
  }
  if (gi != 0) return;
  __syncthreads();
  if (tid == 0) {
    if (err & 1) set_status(a.dev_status, SV_DEV_BAD_TREE);
    else if (err & 2) set_status(a.dev_status, SV_DEV_BAD_TOKEN);
    else if (err & 4) set_status(a.dev_status, SV_DEV_NONFINITE);
    else if (err & 8) set_status(a.dev_status, SV_DEV_TIMEOUT);
    a.accepted_len[b] = err ? -1 : depth;
  }
  for (int j = tid; j <= K; j += TNT) {
    int e = -1, p = -1;
    if (!err && j <= depth) {
      p = s_path[j];
      e = j < depth ? s_tok[s_path[j + 1]] : final_tok;
    }
    a.emitted[trow0 + j] = e;
    if (a.path) a.path[trow0 + j] = p;
  }
  if (a.fin.acc && arrive_last(a.done_cnt, a.B, &flag)) finalize_block(a.fin);
}

}  // namespace

hipError_t launch_init(int32_t *zero_i32, size_t n_i32, int32_t *dev_status, hipStream_t st) {
  const long n = (long)n_i32;
  long blocks = (n + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_init, dim3((unsigned)blocks), dim3(256), 0, st, zero_i32, n, dev_status);
  return hipGetLastError();
}

hipError_t launch_accept_sample(const AcceptArgs &a, hipStream_t st) {
  const size_t shm = sizeof(float) * (2 * a.K + 2);
  const int nw = min(16, max(1, 2 * a.K + 1));
  hipLaunchKernelGGL(k_accept_sample, dim3(a.B), dim3(64 * nw), shm, st, a);
  return hipGetLastError();
}

hipError_t launch_accept_greedy(const AcceptArgs &a, hipStream_t st) {
  const size_t shm = sizeof(int) * (a.K + 2);
  const int nw = min(16, max(1, 2 * (a.K + 1)));  // two waves per row when K + 1 <= 8
  hipLaunchKernelGGL(k_accept_greedy, dim3(a.B), dim3(64 * nw), shm, st, a);
  return hipGetLastError();
}

int sample_chunks(int V) {
  // chunks of at most NT * PER tokens; at most NT chunks (one per thread of the pick)
  int c = (V + NT * PER - 1) / (NT * PER);
  if (c < 1) c = 1;
  return c;
}

hipError_t launch_sample(const SampleJob *jobs, int njobs, int V, float invT, float *chunk_sums, int32_t *out,
                         int32_t *job_cnt, int32_t *done_cnt, const FinalizeArgs &fin, hipStream_t st) {
  (void)job_cnt;
  (void)done_cnt;
  if (njobs <= 0) return hipSuccess;
  const int C = sample_chunks(V);
  // chunks of a multiple of 64 tokens (at most NT * PER): 16-byte aligned when V % 4 == 0
  const int chunk = (((V + C - 1) / C) + 63) / 64 * 64;
  const dim3 grid((C + SUBS - 1) / SUBS, njobs);
  if (V % 4 == 0) {
    hipLaunchKernelGGL(k_sample_sums<true>, grid, dim3(NT), 0, st, jobs, V, chunk, C, invT, chunk_sums);
    hipLaunchKernelGGL(k_sample_pick<true>, dim3(njobs), dim3(T2_NT2), 0, st, jobs, V, chunk, C, invT,
                       (const float *)chunk_sums, out, fin);
  } else {
    hipLaunchKernelGGL(k_sample_sums<false>, grid, dim3(NT), 0, st, jobs, V, chunk, C, invT, chunk_sums);
    hipLaunchKernelGGL(k_sample_pick<false>, dim3(njobs), dim3(T2_NT2), 0, st, jobs, V, chunk, C, invT,
                       (const float *)chunk_sums, out, fin);
  }
  return hipGetLastError();
}

hipError_t launch_tail_small(const AcceptArgs &a, float *sums, float *req, const FinalizeArgs &fin,
                             hipStream_t st) {
  const int C = sample_chunks(a.V);
  // chunks of a multiple of 64 tokens (at most NT * PER = 2048): 16-byte aligned when V % 4 == 0
  const int chunk = (((a.V + C - 1) / C) + 63) / 64 * 64;
  const dim3 grid((C + 1) / 2, a.B);
  if (a.V % 4 == 0) {
    hipLaunchKernelGGL(k_tail_a<true>, grid, dim3(TA_NT), 0, st, a, chunk, C, sums, req);
    hipLaunchKernelGGL(k_tail_b<true>, dim3(a.B), dim3(T2_NT2), 0, st, a, chunk, C, (const float *)sums,
                       (const float *)req, fin);
  } else {
    hipLaunchKernelGGL(k_tail_a<false>, grid, dim3(TA_NT), 0, st, a, chunk, C, sums, req);
    hipLaunchKernelGGL(k_tail_b<false>, dim3(a.B), dim3(T2_NT2), 0, st, a, chunk, C, (const float *)sums,
                       (const float *)req, fin);
  }
  return hipGetLastError();
}

hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t st) {
  const int rows = a.B * a.Kmax;
  if (rows > 0)
    hipLaunchKernelGGL(k_row_conf, dim3((rows + (NT / 64) - 1) / (NT / 64)), dim3(NT), 0, st, a.parts_d, a.nslots_d,
                       rows, a.invT, a.conf, a.dev_status, a.diag, a.diag_row0);
  // keys [B*Kmax], histogram [1025], lengths [B]: up to 68 KiB at the largest batch the
  // entry point takes (B <= 8192, B*Kmax <= 8192), above the 64 KiB a launch gets unless
  // the kernel's dynamic LDS limit is raised (once per device)
  const size_t shm = sizeof(int) * ((size_t)a.B * a.Kmax + 1025 + a.B);
  constexpr size_t shm_max = sizeof(int) * (8192 + 1025 + 8192);
  if (shm > shm_max) return hipErrorInvalidValue;
  if (shm > 65536) {
    static std::atomic<unsigned long long> attr_set{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = 1ull << (dev & 63);
    if (!(attr_set.load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_schedule), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)shm_max);
      if (e != hipSuccess) return e;
      attr_set.fetch_or(bit, std::memory_order_release);
    }
  }
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(1024), shm, st, a);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t *src, uint16_t *dst, const int32_t *row_map, const int32_t *m_total,
                              int max_rows, int d, hipStream_t st) {
  hipLaunchKernelGGL(k_gather_rows, dim3(max_rows), dim3(256), 0, st, src, dst, row_map, m_total, d);
  return hipGetLastError();
}

hipError_t launch_scatter_logits(const float *packed, float *dst, const int32_t *row_map, const int32_t *m_total,
                                 int max_rows, int V, hipStream_t st) {
  hipLaunchKernelGGL(k_scatter_f32, dim3(max_rows), dim3(256), 0, st, packed, dst, row_map, m_total, V);
  return hipGetLastError();
}

hipError_t launch_scatter_hidden(const uint16_t *packed, uint16_t *dst, const int32_t *row_map,
                                 const int32_t *m_total, int max_rows, int d, hipStream_t st) {
  hipLaunchKernelGGL(k_scatter_u16, dim3(max_rows), dim3(256), 0, st, packed, dst, row_map, m_total, d);
  return hipGetLastError();
}

hipError_t launch_propose_finish(const StatPart *parts, int nslots, int rows, float invT, float T,
                                 const float *logits, int V, const float *coins, SampleJob *jobs, int32_t *draft_out,
                                 float *conf_out, int32_t *dev_status, int32_t *job_cnt, hipStream_t st) {
  const int blocks = (rows + (NT / 64) - 1) / (NT / 64);
  hipLaunchKernelGGL(k_propose_finish, dim3(blocks), dim3(NT), 0, st, parts, nslots, rows, invT, T, logits, V,
                     coins, jobs, draft_out, conf_out, dev_status, job_cnt);
  return hipGetLastError();
}

int tree_chunks(int V) { return (V + TCH - 1) / TCH; }

hipError_t launch_tree(const TreeArgs &a, hipStream_t st) {
  // 16-byte loads of logit rows need every row start 16-byte aligned: V % 4 == 0
  const bool vec = a.V % 4 == 0 && (reinterpret_cast<uintptr_t>(a.logits_t) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.logits_d) & 15) == 0;
  if (!a.greedy && a.chunk_sums && a.partials && a.meet) {
    // all B * G blocks resident at once (one per CU at most): a cooperative launch
    // guarantees it or fails, and then the one-block kernel runs instead
    int G = num_cus() / a.B;
    if (G > TREE_MAX_BLOCKS) G = TREE_MAX_BLOCKS;
    if (G >= 2) {
      TreeArgs ac = a;
      void *args[] = {&ac, &G};
      const void *fn = vec ? reinterpret_cast<const void *>(&k_tree_coop<true>)
                           : reinterpret_cast<const void *>(&k_tree_coop<false>);
      if (hipLaunchCooperativeKernel(fn, dim3(a.B * G), dim3(TNT), args, 0, st) == hipSuccess) return hipSuccess;
      (void)hipGetLastError();
    }
  }
  if (vec)
    hipLaunchKernelGGL(k_tree<true>, dim3(a.B), dim3(TNT), 0, st, a);
  else
    hipLaunchKernelGGL(k_tree<false>, dim3(a.B), dim3(TNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
