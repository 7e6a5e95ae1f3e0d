// Host side of libspecverify: argument checks, workspace plan, kernel choice and
// the launch sequence of each verification mode.  Everything is enqueued on the
// caller's stream; there is no host synchronisation and no allocation.
#include <math.h>
#include <mutex>

#include "sv_internal.h"

#define SV_API extern "C" __attribute__((visibility("default")))

namespace sv {

int num_cus() {
  static int cus = 0;
  static std::once_flag once;
  std::call_once(once, [] {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess &&
        p.multiProcessorCount > 0)
      cus = p.multiProcessorCount;
    else
      cus = 256;  // MI355X
    (void)hipGetLastError();
  });
  return cus;
}

namespace {

constexpr size_t ALIGN = 256;
// Up to this many (request, position) candidates the sampled modes draw every possible
// final token speculatively and decide acceptance in the same kernel (latency path).
constexpr int SMALL_TAIL_JOBS = 32;
size_t up(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }

struct Gemm {
  bool stream = true;
  int grid = 0;                     // stream kernel
  TileShape shape{128, 128, 64, 2};  // tiled kernel
  int splits = 1;
  int nslots = 0;  // statistics slots per row (EPI_LOGITS)
  size_t partial_floats = 0;
  // EPI_LOGITS / EPI_SWIGLU: output columns [0, n_split) in whole rounds of `shape` tiles
  // over the CUs, the rest in a second launch of `shape2` tiles (0: one launch)
  int n_split = 0;
  TileShape shape2{256, 128, 64, 3};
};

Gemm choose(int M, int N, int K, int epi) {
  Gemm g;
  if (stream_ok(M, epi)) {
    g.stream = true;
    const int ntiles = (N + 15) / 16;
    g.grid = ntiles < num_cus() ? ntiles : num_cus();
    g.nslots = g.grid;
    return g;
  }
  g.stream = false;
  g.shape = tiled_shape(M, N, K, epi);
  const int Ncols = epi == EPI_SWIGLU ? 2 * N : N;
  const long tiles = (long)((M + g.shape.bm - 1) / g.shape.bm) * ((Ncols + g.shape.bn - 1) / g.shape.bn);
  // the down projection (few output columns, long K) splits K until the tiles fill the
  // resident workgroup slots; split SwiGLU and logits tiles measured slower
  const long slots = (long)tiled_per_cu(g.shape) * num_cus();
  if (epi == EPI_RESID && tiles < slots) {
    const int want = (int)((slots + tiles - 1) / tiles);
    int maxs = (K / g.shape.bk) / 4;
    if (maxs > 8) maxs = 8;
    if (maxs < 1) maxs = 1;
    g.splits = want < maxs ? want : maxs;
  }
  if (g.splits > 1) g.partial_floats = (size_t)g.splits * M * Ncols;
  if (epi == EPI_SWIGLU && M > 192) {
    // Whole rounds of 256 x 256 tiles, then the remaining output columns as one launch of
    // 256 x 128 tiles, when that costs less than either shape alone (a 256 x 256 tile
    // takes ~1.7-1.9x a 256 x 128 one): 1024 rows at d_ff = 12288 run 1 + 1 rounds
    // (126 + 70 us) instead of 3 rounds of 256 x 128 tiles (204 us).
    const long tm = (M + 255) / 256, cus = num_cus();
    const long tiles256 = tm * ((2L * N + 255) / 256);
    const long full = tiles256 / cus;
    if (full >= 1 && tiles256 % cus > 0 && cus % tm == 0) {
      const long n1 = full * (cus / tm) * 128;  // output columns of the whole rounds
      if (n1 < N) {
        const long r2 = (tm * ((2L * (N - n1) + 127) / 128) + cus - 1) / cus;
        const long r128 = (tm * ((2L * N + 127) / 128) + cus - 1) / cus;
        const long r256 = (tiles256 + cus - 1) / cus;
        const long best = 10 * r128 < 17 * r256 ? 10 * r128 : 17 * r256;
        if (17 * full + 10 * r2 < best) {
          g.shape = TileShape{256, 256, 64, 2};
          g.shape2 = TileShape{256, 128, 64, 3};
          g.n_split = (int)n1;
        }
      }
    }
  }
  if (epi == EPI_LOGITS) {
    g.nslots = tiled_slots(N, g.shape);
    // A last round of 256 x 256 tiles at most half full would cost a whole round: its
    // columns go to a second launch of 256 x 128 tiles that fits in one round (half the
    // work per tile).  Measured at 1024 rows: 9.28 rounds -> 9 + one half-size round.
    const TileShape big{256, 256, 64, 2};
    if (g.shape.bm == big.bm && g.shape.bn == big.bn && g.shape.bk == big.bk && g.shape.ns == big.ns) {
      const long tm = (M + 255) / 256, nt = (N + 255) / 256;
      const long full = tiles / slots, rem = tiles % slots;
      if (full >= 1 && rem > 0 && 2 * rem <= slots && slots % tm == 0) {
        const long n1 = full * (slots / tm) * 256;
        const long tiles2 = tm * ((N - n1 + 127) / 128);
        if (n1 < N && nt * tm == tiles && tiles2 <= (long)tiled_per_cu(g.shape2) * num_cus()) {
          g.n_split = (int)n1;
          g.nslots = tiled_slots((int)n1, g.shape) + tiled_slots(N - (int)n1, g.shape2);
        }
      }
    }
  }
  return g;
}

struct Plan {
  int mode = 0, B = 0, K = 0, d = 0, d_ff = 0, V = 0;
  int M_t = 0, M_lm = 0, rows_d = 0, budget = 0;
  Gemm gu, dn, lm, s1;
  // scheduled mode: plans for at most m_split verified rows (gu_lo, dn_lo, lm_lo), run
  // beside the budget-sized plans; the device-side row count picks the one that works
  int m_split = 0;
  Gemm gu_lo, dn_lo, lm_lo;
  size_t o_a = 0, o_y = 0, o_part = 0, o_parts = 0, o_parts_d = 0, o_logits = 0, o_logits_d = 0,
         o_jobs = 0, o_sums = 0, o_conf = 0, o_vlen = 0, o_rowoff = 0, o_rowmap = 0, o_mtot = 0,
         o_hp = 0, o_sync = 0, o_lse = 0, o_tree = 0, o_nslots = 0, total = 0;
  bool small_tail = false;  // B*(K+1) <= 32: acceptance in every chunk block, then the draw
};

bool valid_weights(const sv_weights *w) {
  if (!w || !w->w_lm) return false;
  if (w->wtype != SV_WEIGHTS_BF16 && w->wtype != SV_WEIGHTS_FP8_E4M3) return false;
  if (w->wtype == SV_WEIGHTS_FP8_E4M3) {
    if (!w->s_lm) return false;
    if (w->d_ff > 0 && (!w->s_gate || !w->s_up || !w->s_down)) return false;
  }
  if (w->d <= 0 || (w->d % 64) != 0) return false;
  if (w->V < 1 || w->V > (1 << 19)) return false;  // sampling keeps at most 256 chunks of 2048 tokens
  if (w->d_ff < 0 || (w->d_ff % 64) != 0) return false;
  const bool has = w->d_ff > 0;
  if (has != (w->w_gate != nullptr) || has != (w->w_up != nullptr) || has != (w->w_down != nullptr)) return false;
  return true;
}

// FP8 weights run on the weight-streaming kernel only, which stages the row scales of
// a workgroup's whole column range (at most 2048 columns).
bool fp8_ok(const Gemm &g, int N) {
  if (!g.stream || g.grid < 1) return false;
  const int ntiles = (N + 15) / 16;
  return 16 * ((ntiles + g.grid - 1) / g.grid) <= 2048;
}

// Scheduled mode: the verified rows are known only on the device, and the budget-sized
// plans (256-row tiles at a 512-row budget) run far below their rate when few rows pass
// the threshold.  Plans for at most SMALL_ROWS rows are kept beside them when the
// budget-sized LM head uses taller tiles; both are launched and the device-side count
// lets exactly one of each pair work.  The LM-head launch that works writes its plan's
// statistics slot count for the acceptance kernel, so the two plans may tile the
// columns differently.
constexpr int SMALL_ROWS = 128;

// LM head for at most SMALL_ROWS rows: whole rounds of 128 x 256 tiles over the CUs, the
// remaining columns as 128 x 128 tiles in a second launch (a last round of 256-column
// tiles a third full would cost nearly a whole round).
Gemm small_lm_plan(int V, int d) {
  Gemm g = choose(SMALL_ROWS, V, d, EPI_LOGITS);
  if (g.stream) return g;
  const TileShape wide{128, 256, 64, 3}, narrow{128, 128, 64, 4};
  const long slots = (long)tiled_per_cu(wide) * num_cus();
  const long tiles = (V + 255) / 256;
  const long full = slots > 0 ? tiles / slots : 0;
  g.shape = wide;
  g.n_split = 0;
  g.nslots = tiled_slots(V, wide);
  if (full >= 1 && tiles % slots > 0) {
    const long n1 = full * slots * 256;
    if (n1 < V) {
      g.n_split = (int)n1;
      g.shape2 = narrow;
      g.nslots = tiled_slots((int)n1, wide) + tiled_slots(V - (int)n1, narrow);
    }
  }
  return g;
}

bool plan_small_rows(Plan &p, int V) {
  if (p.budget <= SMALL_ROWS || p.lm.stream || p.lm.shape.bm <= SMALL_ROWS) return false;
  const Gemm lo = small_lm_plan(V, p.d);
  if (lo.stream) return false;
  if (p.d_ff > 0) {
    p.gu_lo = choose(SMALL_ROWS, p.d_ff, p.d, EPI_SWIGLU);
    p.dn_lo = choose(SMALL_ROWS, p.d, p.d_ff, EPI_RESID);
    if (p.gu_lo.stream || p.dn_lo.stream || p.gu.stream || p.dn.stream) return false;
  }
  p.lm_lo = lo;
  p.m_split = SMALL_ROWS;
  return true;
}

bool make_plan(int mode, int B, int K, const sv_weights *w, int budget, Plan &p) {
  if (!valid_weights(w) || B < 1 || K < 0) return false;
  if ((long)B * (K + 1) >= (1L << 31) / 2) return false;
  p.mode = mode; p.B = B; p.K = K; p.d = w->d; p.d_ff = w->d_ff; p.V = w->V;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += up(bytes); return o; };
  const int d = w->d, V = w->V;
  if (mode == SV_MODE_PROPOSE) {
    p.M_lm = B;
    p.lm = choose(B, V, d, EPI_LOGITS);
    p.o_parts = take(sizeof(StatPart) * (size_t)B * p.lm.nslots);
    p.o_logits = take(sizeof(float) * (size_t)B * V);
    p.o_jobs = take(sizeof(SampleJob) * (size_t)B);
    p.o_sums = take(sizeof(float) * 2 * (size_t)B * sample_chunks(V));
    p.o_sync = take(sizeof(int32_t) * (size_t)(B + 1));
    p.total = off;
    return w->wtype != SV_WEIGHTS_FP8_E4M3 || fp8_ok(p.lm, V);
  }
  int M_mlp;
  if (mode == SV_MODE_SCHEDULED) {
    if (budget < B) return false;
    p.budget = budget;
    p.rows_d = B * K;
    M_mlp = budget < B * (K + 1) ? budget : B * (K + 1);
    p.budget = M_mlp;
    p.M_t = M_mlp;
    p.M_lm = M_mlp;
  } else {
    p.M_t = B * (K + 1);
    p.rows_d = B * K;
    M_mlp = p.M_t;
    p.M_lm = mode == SV_MODE_SAMPLE ? p.M_t + p.rows_d : p.M_t;
  }
  size_t part_floats = 0;
  if (w->d_ff > 0) {
    p.gu = choose(M_mlp, w->d_ff, d, EPI_SWIGLU);
    p.dn = choose(M_mlp, d, w->d_ff, EPI_RESID);
    part_floats = p.gu.partial_floats > p.dn.partial_floats ? p.gu.partial_floats : p.dn.partial_floats;
    p.o_a = take(2 * (size_t)M_mlp * w->d_ff);
    p.o_y = take(2 * (size_t)M_mlp * d);
  }
  p.lm = choose(p.M_lm, V, d, EPI_LOGITS);
  if (mode == SV_MODE_SCHEDULED && w->wtype == SV_WEIGHTS_BF16 && plan_small_rows(p, V)) {
    if (p.gu_lo.partial_floats > part_floats) part_floats = p.gu_lo.partial_floats;
    if (p.dn_lo.partial_floats > part_floats) part_floats = p.dn_lo.partial_floats;
  }
  if (part_floats) p.o_part = take(sizeof(float) * part_floats);
  const int nslots_max = p.m_split > 0 && p.lm_lo.nslots > p.lm.nslots ? p.lm_lo.nslots : p.lm.nslots;
  p.o_parts = take(sizeof(StatPart) * (size_t)p.M_lm * nslots_max);
  const int NJ = B * (K + 1);
  if (mode != SV_MODE_GREEDY) {
    p.small_tail = NJ <= SMALL_TAIL_JOBS;
    p.o_logits = take(sizeof(float) * (size_t)p.M_lm * V);
    p.o_jobs = take(sizeof(SampleJob) * (size_t)B);
    p.o_sums = take(sizeof(float) * 2 * (size_t)B * sample_chunks(V));  // per request: chunk sums
    if (p.small_tail) p.o_lse = take(sizeof(float) * 3 * (size_t)B);  // per request: A, normalisers
    // sampled tree verification over several blocks per request: chunk sums and slice totals
    if (mode == SV_MODE_SAMPLE)
      p.o_tree = take(sizeof(float) * ((size_t)B * tree_chunks(V) + (size_t)B * 2 * TREE_MAX_BLOCKS));
  }
  // arrival counters: [0] call-wide, [1 + i] per request (or per candidate job)
  p.o_sync = take(sizeof(int32_t) * (size_t)(1 + (p.small_tail ? NJ : B)));
  if (mode == SV_MODE_SCHEDULED) {
    p.s1 = choose(p.rows_d > 0 ? p.rows_d : 1, V, d, EPI_LOGITS);
    p.o_parts_d = take(sizeof(StatPart) * (size_t)(p.rows_d > 0 ? p.rows_d : 1) * p.s1.nslots);
    p.o_logits_d = take(sizeof(float) * (size_t)(p.rows_d > 0 ? p.rows_d : 1) * V);
    p.o_conf = take(sizeof(float) * (size_t)(p.rows_d > 0 ? p.rows_d : 1));
    p.o_vlen = take(sizeof(int32_t) * (size_t)B);
    p.o_rowoff = take(sizeof(int32_t) * (size_t)(B + 1));
    p.o_rowmap = take(sizeof(int32_t) * (size_t)p.budget);
    p.o_mtot = take(sizeof(int32_t));
    p.o_nslots = take(sizeof(int32_t));
    p.o_hp = take(2 * (size_t)p.budget * d);
  }
  p.total = off;
  if (w->wtype == SV_WEIGHTS_FP8_E4M3) {
    if (!fp8_ok(p.lm, V)) return false;
    if (w->d_ff > 0 && (!fp8_ok(p.gu, w->d_ff) || !fp8_ok(p.dn, d))) return false;
    if (mode == SV_MODE_SCHEDULED && p.rows_d > 0 && !fp8_ok(p.s1, V)) return false;
  }
  return true;
}

bool aligned16(const void *q) { return ((uintptr_t)q & 15u) == 0; }

template <typename T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off); }

thread_local const char *g_last_hip_error = "no error";

#define SV_CHECK(expr)                                  \
  do {                                                  \
    const hipError_t e_ = (expr);                       \
    if (e_ != hipSuccess) {                             \
      g_last_hip_error = hipGetErrorString(e_);         \
      (void)hipGetLastError();                          \
      return SV_EHIP;                                   \
    }                                                   \
  } while (0)

hipError_t run_gemm(const Gemm &g, GemmArgs a, int epi, hipStream_t st) {
  if (g.stream) return launch_gemm_stream(a, epi, g.grid, st);
  if (g.n_split > 0) {  // two launches over disjoint ranges of output columns
    GemmArgs a1 = a;
    a1.N = g.n_split;
    hipError_t e = launch_gemm_tiled(a1, epi, g.shape, 1, st);
    if (e != hipSuccess) return e;
    GemmArgs a2 = a;
    a2.N = a.N - g.n_split;
    a2.w = a.w + (size_t)g.n_split * a.K;
    if (epi == EPI_SWIGLU) {
      a2.w2 = a.w2 + (size_t)g.n_split * a.K;
      a2.out = a.out + g.n_split;
    } else {
      if (a.logits) a2.logits = a.logits + g.n_split;
      a2.parts = a.parts + tiled_slots(g.n_split, g.shape);
      a2.n_off = a.n_off + g.n_split;
    }
    a2.status_reset = nullptr;
    a2.counter_reset = nullptr;
    a2.nslots_out = nullptr;
    return launch_gemm_tiled(a2, epi, g.shape2, 1, st);
  }
  if (g.splits > 1) {
    hipError_t e = launch_gemm_tiled(a, epi, g.shape, g.splits, st);
    if (e != hipSuccess) return e;
    return launch_splitk_reduce(a, epi, g.splits, g.shape.bn, st);
  }
  return launch_gemm_tiled(a, epi, g.shape, 1, st);
}

// The dominant GEMM of a call, bracketed by the caller's optional measurement events.
hipError_t run_gemm_timed(const Gemm &g, const GemmArgs &a, int epi, const sv_outputs *out, hipStream_t st) {
  if (out->ev_lm_begin) {
    hipError_t e = hipEventRecord((hipEvent_t)out->ev_lm_begin, st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = run_gemm(g, a, epi, st);
  if (e != hipSuccess) return e;
  if (out->ev_lm_end) return hipEventRecord((hipEvent_t)out->ev_lm_end, st);
  return hipSuccess;
}

GemmArgs base_args() {
  GemmArgs a = {};
  a.invT = 1.f;
  return a;
}

// S3 + S4: a = bf16(silu(h W_gate^T) * (h W_up^T)), y = bf16(h + a W_down^T).
// Weights of one product: bf16 bit patterns, or FP8 codes and their row scales.
void set_w(GemmArgs &g, const void *wt, const float *sc, const void *wt2, const float *sc2, int32_t wtype) {
  g.w = static_cast<const uint16_t *>(wt);
  g.w2 = static_cast<const uint16_t *>(wt2);
  g.wfp8 = wtype == SV_WEIGHTS_FP8_E4M3;
  g.wscale = g.wfp8 ? sc : nullptr;
  g.wscale2 = g.wfp8 ? sc2 : nullptr;
}
void set_lm(GemmArgs &g, const sv_weights *w) { set_w(g, w->w_lm, w->s_lm, nullptr, nullptr, w->wtype); }

// With a device-side row count M_dev, the pair of launches does its work only when
// m_lo < *M_dev <= m_hi (m_hi = 0: no upper limit).
hipError_t run_mlp_plans(const Plan &p, const Gemm &gu, const Gemm &dnp, const sv_weights *w, const uint16_t *h,
                         int M, const int *M_dev, int m_lo, int m_hi, uint16_t *y, void *ws, int32_t *status_reset,
                         hipStream_t st) {
  uint16_t *abuf = at<uint16_t>(ws, p.o_a);
  GemmArgs g = base_args();
  g.x1 = h; g.ldx1 = p.d; g.m1 = M; g.x2 = h; g.ldx2 = p.d;
  g.M = M; g.M_dev = M_dev; g.m_lo = m_lo; g.m_hi = m_hi; g.N = p.d_ff; g.K = p.d;
  set_w(g, w->w_gate, w->s_gate, w->w_up, w->s_up, w->wtype);
  g.out = abuf; g.ldo = p.d_ff;
  g.partial = gu.splits > 1 ? at<float>(ws, p.o_part) : nullptr;
  g.status_reset = status_reset;
  hipError_t e = run_gemm(gu, g, EPI_SWIGLU, st);
  if (e != hipSuccess) return e;
  GemmArgs dn = base_args();
  dn.x1 = abuf; dn.ldx1 = p.d_ff; dn.m1 = M; dn.x2 = abuf; dn.ldx2 = p.d_ff;
  dn.M = M; dn.M_dev = M_dev; dn.m_lo = m_lo; dn.m_hi = m_hi; dn.N = p.d; dn.K = p.d_ff;
  set_w(dn, w->w_down, w->s_down, nullptr, nullptr, w->wtype);
  dn.out = y; dn.ldo = p.d; dn.resid = h; dn.ldr = p.d;
  dn.partial = dnp.splits > 1 ? at<float>(ws, p.o_part) : nullptr;
  return run_gemm(dnp, dn, EPI_RESID, st);
}

hipError_t run_mlp(const Plan &p, const sv_weights *w, const uint16_t *h, int M, const int *M_dev, uint16_t *y,
                   void *ws, int32_t *status_reset, hipStream_t st) {
  return run_mlp_plans(p, p.gu, p.dn, w, h, M, M_dev, 0, 0, y, ws, status_reset, st);
}

int check_common(const sv_weights *w, const uint16_t *h, const int32_t *draft, int B, int K, void *ws,
                 const sv_outputs *out) {
  if (!valid_weights(w) || !h || B < 1 || K < 0 || !out) return SV_EINVAL;
  // the acceptance kernels keep a request's row normalisers in LDS: 2 K + 2 floats,
  // within the 64 KiB a launch gets
  if (K > SV_MAX_K) return SV_EINVAL;
  if (K > 0 && !draft) return SV_EINVAL;
  if (!out->accepted_len || !out->emitted || !out->tau) return SV_EINVAL;
  if (!aligned16(h) || !aligned16(w->w_lm)) return SV_EINVAL;
  if (w->d_ff > 0 && (!aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down))) return SV_EINVAL;
  if (ws && ((uintptr_t)ws & (ALIGN - 1))) return SV_EINVAL;
  return SV_OK;
}

}  // namespace
}  // namespace sv

using namespace sv;

SV_API size_t sv_workspace_bytes(int mode, int B, int K, const sv_weights *w) {
  Plan p;
  if (mode < SV_MODE_GREEDY || mode > SV_MODE_PROPOSE) return 0;
  const int budget = mode == SV_MODE_SCHEDULED ? B * (K + 1) : 0;
  if (!make_plan(mode, B, K, w, budget, p)) return 0;
  return p.total ? p.total : ALIGN;
}

SV_API int spec_verify_greedy(const sv_weights *w, const uint16_t *h, const int32_t *draft, int B, int K, void *ws,
                              size_t ws_bytes, sv_outputs *out, void *stream) {
  int rc = check_common(w, h, draft, B, K, ws, out);
  if (rc) return rc;
  Plan p;
  if (!make_plan(SV_MODE_GREEDY, B, K, w, 0, p)) return SV_EINVAL;
  if (ws_bytes < p.total || (p.total && !ws)) return SV_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  int32_t *reset = out->dev_status;
  const uint16_t *y = h;
  if (p.d_ff > 0) {
    uint16_t *ybuf = out->hidden ? out->hidden : at<uint16_t>(ws, p.o_y);
    SV_CHECK(run_mlp(p, w, h, p.M_t, nullptr, ybuf, ws, reset, st));
    reset = nullptr;
    y = ybuf;
  }
  GemmArgs g = base_args();
  g.x1 = y; g.ldx1 = p.d; g.m1 = p.M_t; g.x2 = y; g.ldx2 = p.d;
  g.M = p.M_t; g.N = p.V; g.K = p.d; set_lm(g, w);
  g.logits = out->logits; g.ldl = p.V;
  g.parts = at<StatPart>(ws, p.o_parts); g.nslots = p.lm.nslots;
  g.invT = 1.f; g.want_s = out->diag ? 1 : 0;
  g.status_reset = reset;
  int32_t *sync = at<int32_t>(ws, p.o_sync);
  g.counter_reset = sync;
  SV_CHECK(run_gemm_timed(p.lm, g, EPI_LOGITS, out, st));
  AcceptArgs a = {};
  a.B = B; a.K = K; a.V = p.V; a.invT = 1.f;
  a.parts_t = g.parts; a.nslots_t = p.lm.nslots;
  a.logits_t = out->logits;
  a.draft = draft; a.accepted_len = out->accepted_len; a.emitted = out->emitted;
  a.dev_status = out->dev_status; a.diag = out->diag;
  a.done_cnt = sync;
  a.fin = FinalizeArgs{out->accepted_len, nullptr, B, K, out->tau, out->counters};
  SV_CHECK(launch_accept_greedy(a, st));
  return SV_OK;
}

SV_API int spec_verify_sample(const sv_weights *w, const uint16_t *h, const uint16_t *h_draft, const int32_t *draft,
                              const float *u, float T, int B, int K, void *ws, size_t ws_bytes, sv_outputs *out,
                              void *stream) {
  int rc = check_common(w, h, draft, B, K, ws, out);
  if (rc) return rc;
  if (!u || !(T > 0.f) || !isfinite(T)) return SV_EINVAL;
  if (K > 0 && (!h_draft || !aligned16(h_draft))) return SV_EINVAL;
  Plan p;
  if (!make_plan(SV_MODE_SAMPLE, B, K, w, 0, p)) return SV_EINVAL;
  if (ws_bytes < p.total || !ws) return SV_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const float invT = 1.f / T;
  int32_t *reset = out->dev_status;
  const uint16_t *y = h;
  if (p.d_ff > 0) {
    uint16_t *ybuf = out->hidden ? out->hidden : at<uint16_t>(ws, p.o_y);
    SV_CHECK(run_mlp(p, w, h, p.M_t, nullptr, ybuf, ws, reset, st));
    reset = nullptr;
    y = ybuf;
  }
  float *logits = out->logits ? out->logits : at<float>(ws, p.o_logits);
  GemmArgs g = base_args();
  g.x1 = y; g.ldx1 = p.d; g.m1 = p.M_t; g.x2 = K > 0 ? h_draft : y; g.ldx2 = p.d;
  g.M = p.M_lm; g.N = p.V; g.K = p.d; set_lm(g, w);
  g.logits = logits; g.ldl = p.V;
  g.parts = at<StatPart>(ws, p.o_parts); g.nslots = p.lm.nslots;
  g.invT = invT; g.want_s = 1;
  g.status_reset = reset;
  int32_t *sync = at<int32_t>(ws, p.o_sync);
  SV_CHECK(run_gemm_timed(p.lm, g, EPI_LOGITS, out, st));
  AcceptArgs a = {};
  a.B = B; a.K = K; a.V = p.V; a.invT = invT;
  a.parts_t = g.parts; a.nslots_t = p.lm.nslots;
  a.parts_d = g.parts + (size_t)p.M_t * p.lm.nslots; a.nslots_d = p.lm.nslots;
  a.logits_t = logits; a.logits_d = logits + (size_t)p.M_t * p.V;
  a.draft = draft; a.u = u;
  a.accepted_len = out->accepted_len; a.emitted = out->emitted;
  a.jobs = at<SampleJob>(ws, p.o_jobs);
  a.dev_status = out->dev_status; a.diag = out->diag;
  a.done_cnt = sync; a.job_cnt = sync + 1;
  const FinalizeArgs fin{out->accepted_len, nullptr, B, K, out->tau, out->counters};
  if (p.small_tail) {
    SV_CHECK(launch_tail_small(a, at<float>(ws, p.o_sums), at<float>(ws, p.o_lse), fin, st));
    return SV_OK;
  }
  SV_CHECK(launch_accept_sample(a, st));
  SV_CHECK(launch_sample(a.jobs, B, p.V, invT, at<float>(ws, p.o_sums), out->emitted, sync + 1, sync, fin, st));
  return SV_OK;
}

// ---- the sampled verification without any allocation: the workspace is the file-scope
// device array below (one copy per GPU, kept until the process ends)
namespace sv {
namespace {
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)SV_STATIC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];  // device address of `scratch` on each device, once looked up
}  // namespace
}  // namespace sv

static __device__ __align__(256) uint8_t scratch[sv::STATIC_SCRATCH_BYTES];

SV_API int spec_verify_sample_noalloc(const sv_weights *w, const uint16_t *h, const uint16_t *h_draft,
                                      const int32_t *draft, const float *u, float T, int B, int K, sv_outputs *out,
                                      void *stream) {
  // every argument is checked before the first device call
  int rc = check_common(w, h, draft, B, K, nullptr, out);
  if (rc) return rc;
  if (!u || !(T > 0.f) || !isfinite(T)) return SV_EINVAL;
  if (K > 0 && (!h_draft || !aligned16(h_draft))) return SV_EINVAL;
  Plan p;
  if (!make_plan(SV_MODE_SAMPLE, B, K, w, 0, p)) return SV_EINVAL;
  if (p.total > STATIC_SCRATCH_BYTES) return SV_ESCRATCH;
  int dev = 0;
  SV_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= MAX_DEVICES) return SV_EINVAL;
  void *ptr;
  {
    // The array's name is a host-side stand-in: its device address is looked up once per
    // device, with that device current, and only that address is handed to the kernels.
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void *q = nullptr;
      SV_CHECK(hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)));
      if (!q) return SV_EHIP;
      g_scratch_ptr[dev] = q;
    }
    ptr = g_scratch_ptr[dev];
  }
  return spec_verify_sample(w, h, h_draft, draft, u, T, B, K, ptr, STATIC_SCRATCH_BYTES, out, stream);
}

SV_API int spec_verify_scheduled(const sv_weights *w, const uint16_t *h, const uint16_t *h_draft,
                                 const int32_t *draft, const float *u, float T, float survival_threshold,
                                 int budget_rows, int B, int Kmax, void *ws, size_t ws_bytes, sv_outputs *out,
                                 void *stream) {
  int rc = check_common(w, h, draft, B, Kmax, ws, out);
  if (rc) return rc;
  if (!u || !(T > 0.f) || !isfinite(T)) return SV_EINVAL;
  if (!(survival_threshold > 0.f) || !(survival_threshold <= 1.f)) return SV_EINVAL;
  if (budget_rows < B || B > 8192 || (long)B * Kmax > 8192) return SV_EINVAL;
  if (Kmax > 0 && (!h_draft || !aligned16(h_draft))) return SV_EINVAL;
  Plan p;
  if (!make_plan(SV_MODE_SCHEDULED, B, Kmax, w, budget_rows, p)) return SV_EINVAL;
  if (ws_bytes < p.total || !ws) return SV_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const float invT = 1.f / T;
  const int rows_d = B * Kmax;
  float *logits_d = (out->logits && rows_d) ? out->logits + (size_t)B * (Kmax + 1) * p.V : at<float>(ws, p.o_logits_d);
  StatPart *parts_d = at<StatPart>(ws, p.o_parts_d);
  int32_t *vlen = at<int32_t>(ws, p.o_vlen);
  int32_t *rowoff = at<int32_t>(ws, p.o_rowoff);
  int32_t *rowmap = at<int32_t>(ws, p.o_rowmap);
  int32_t *mtot = at<int32_t>(ws, p.o_mtot);
  uint16_t *hp = at<uint16_t>(ws, p.o_hp);
  int32_t *reset = out->dev_status;
  // S1: confidences of every draft row through the shared LM head
  if (rows_d > 0) {
    GemmArgs g = base_args();
    g.x1 = h_draft; g.ldx1 = p.d; g.m1 = rows_d; g.x2 = h_draft; g.ldx2 = p.d;
    g.M = rows_d; g.N = p.V; g.K = p.d; set_lm(g, w);
    g.logits = logits_d; g.ldl = p.V;
    g.parts = parts_d; g.nslots = p.s1.nslots;
    g.invT = invT; g.want_s = 1;
    g.status_reset = reset;
    reset = nullptr;
    SV_CHECK(run_gemm_timed(p.s1, g, EPI_LOGITS, out, st));
  }
  // S2: survival schedule, budget, packing
  ScheduleArgs sa = {};
  sa.B = B; sa.Kmax = Kmax; sa.V = p.V; sa.invT = invT; sa.threshold = survival_threshold;
  sa.budget = p.budget; sa.parts_d = parts_d; sa.nslots_d = p.s1.nslots;
  sa.verify_len = vlen; sa.row_off = rowoff; sa.row_map = rowmap; sa.m_total = mtot;
  sa.conf = at<float>(ws, p.o_conf); sa.dev_status = out->dev_status; sa.verify_len_out = out->verify_len;
  sa.status_reset = reset;
  sa.diag = out->diag;
  sa.diag_row0 = (long)B * (Kmax + 1);
  reset = nullptr;
  SV_CHECK(launch_schedule(sa, st));
  SV_CHECK(launch_gather_rows(h, hp, rowmap, mtot, p.budget, p.d, st));
  // S3-S5 on the packed target rows: with small-row plans, each product is launched for
  // at most m_split rows and for more, and the device-side count m_total picks one
  const int ms = p.m_split;
  const uint16_t *y = hp;
  if (p.d_ff > 0) {
    uint16_t *ybuf = at<uint16_t>(ws, p.o_y);
    if (ms > 0) SV_CHECK(run_mlp_plans(p, p.gu_lo, p.dn_lo, w, hp, ms, mtot, 0, ms, ybuf, ws, nullptr, st));
    SV_CHECK(run_mlp_plans(p, p.gu, p.dn, w, hp, p.budget, mtot, ms, 0, ybuf, ws, nullptr, st));
    y = ybuf;
  }
  float *logits_t = at<float>(ws, p.o_logits);
  GemmArgs g = base_args();
  g.x1 = y; g.ldx1 = p.d; g.m1 = p.budget; g.x2 = y; g.ldx2 = p.d;
  g.M = p.budget; g.M_dev = mtot; g.N = p.V; g.K = p.d; set_lm(g, w);
  g.logits = logits_t; g.ldl = p.V;
  g.parts = at<StatPart>(ws, p.o_parts); g.nslots = p.lm.nslots;
  g.invT = invT; g.want_s = 1;
  int32_t *sync = at<int32_t>(ws, p.o_sync);
  int32_t *nslots_dev = nullptr;
  if (ms > 0) {
    // each plan's launch that works reports its slot count to the acceptance kernel
    nslots_dev = at<int32_t>(ws, p.o_nslots);
    GemmArgs gl = g;
    gl.M = ms; gl.m1 = ms; gl.m_hi = ms;
    gl.nslots = p.lm_lo.nslots;
    gl.nslots_out = nslots_dev; gl.nslots_plan = p.lm_lo.nslots;
    SV_CHECK(run_gemm(p.lm_lo, gl, EPI_LOGITS, st));
    g.m_lo = ms;
    g.nslots_out = nslots_dev; g.nslots_plan = p.lm.nslots;
  }
  SV_CHECK(run_gemm(p.lm, g, EPI_LOGITS, st));
  // S6-S9
  AcceptArgs a = {};
  a.B = B; a.K = Kmax; a.V = p.V; a.invT = invT;
  a.parts_t = g.parts; a.nslots_t = p.lm.nslots; a.nslots_t_dev = nslots_dev;
  a.parts_d = parts_d; a.nslots_d = p.s1.nslots;
  a.logits_t = logits_t; a.logits_d = logits_d;
  a.draft = draft; a.u = u; a.verify_len = vlen; a.row_off = rowoff;
  a.accepted_len = out->accepted_len; a.emitted = out->emitted;
  a.jobs = at<SampleJob>(ws, p.o_jobs);
  a.dev_status = out->dev_status; a.diag = out->diag;
  a.done_cnt = sync; a.job_cnt = sync + 1;
  const FinalizeArgs fin{out->accepted_len, vlen, B, Kmax, out->tau, out->counters};
  if (p.small_tail) {
    SV_CHECK(launch_tail_small(a, at<float>(ws, p.o_sums), at<float>(ws, p.o_lse), fin, st));
  } else {
    SV_CHECK(launch_accept_sample(a, st));
    SV_CHECK(launch_sample(a.jobs, B, p.V, invT, at<float>(ws, p.o_sums), out->emitted, sync + 1, sync, fin, st));
  }
  if (out->logits) SV_CHECK(launch_scatter_logits(logits_t, out->logits, rowmap, mtot, p.budget, p.V, st));
  if (out->hidden && p.d_ff > 0)
    SV_CHECK(launch_scatter_hidden(at<uint16_t>(ws, p.o_y), out->hidden, rowmap, mtot, p.budget, p.d, st));
  return SV_OK;
}

SV_API int spec_draft_propose(const sv_weights *w, const uint16_t *h_draft, const float *coins, float T, int rows,
                              void *ws, size_t ws_bytes, int32_t *draft_out, float *conf_out, void *stream) {
  if (!valid_weights(w) || !h_draft || rows < 1 || !draft_out) return SV_EINVAL;
  if (!(T >= 0.f) || !isfinite(T) || (T > 0.f && !coins)) return SV_EINVAL;
  if (!aligned16(h_draft) || !aligned16(w->w_lm)) return SV_EINVAL;
  if (ws && ((uintptr_t)ws & (ALIGN - 1))) return SV_EINVAL;
  Plan p;
  if (!make_plan(SV_MODE_PROPOSE, rows, 0, w, 0, p)) return SV_EINVAL;
  if (ws_bytes < p.total || !ws) return SV_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const bool samp = T > 0.f;
  const float invT = samp ? 1.f / T : 1.f;
  float *logits = at<float>(ws, p.o_logits);
  GemmArgs g = base_args();
  g.x1 = h_draft; g.ldx1 = p.d; g.m1 = rows; g.x2 = h_draft; g.ldx2 = p.d;
  g.M = rows; g.N = p.V; g.K = p.d; set_lm(g, w);
  g.logits = samp ? logits : nullptr; g.ldl = p.V;
  g.parts = at<StatPart>(ws, p.o_parts); g.nslots = p.lm.nslots;
  g.invT = invT; g.want_s = samp ? 1 : 0;
  SV_CHECK(run_gemm(p.lm, g, EPI_LOGITS, st));
  SampleJob *jobs = at<SampleJob>(ws, p.o_jobs);
  int32_t *sync = at<int32_t>(ws, p.o_sync);
  SV_CHECK(launch_propose_finish(g.parts, p.lm.nslots, rows, invT, T, logits, p.V, coins, jobs, draft_out, conf_out,
                                 nullptr, sync + 1, st));
  if (samp) {
    const FinalizeArgs none{nullptr, nullptr, 0, 0, nullptr, nullptr};
    SV_CHECK(launch_sample(jobs, rows, p.V, invT, at<float>(ws, p.o_sums), draft_out, sync + 1, sync, none, st));
  }
  return SV_OK;
}

SV_API int spec_verify_tree(const sv_weights *w, const uint16_t *h, const uint16_t *h_draft, const int32_t *tokens,
                            const int32_t *parent, const float *u, float T, int B, int K, void *ws, size_t ws_bytes,
                            sv_outputs *out, int32_t *path, int wait_polls, void *stream) {
  int rc = check_common(w, h, tokens, B, K, ws, out);
  if (rc) return rc;
  if (K > 63 || (K > 0 && !parent) || !(T >= 0.f) || !isfinite(T)) return SV_EINVAL;
  const bool greedy = T == 0.f;
  if (!greedy && (!u || (K > 0 && (!h_draft || !aligned16(h_draft))))) return SV_EINVAL;
  Plan p;
  if (!make_plan(greedy ? SV_MODE_GREEDY : SV_MODE_SAMPLE, B, K, w, 0, p)) return SV_EINVAL;
  if (ws_bytes < p.total || (p.total && !ws)) return SV_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const float invT = greedy ? 1.f : 1.f / T;
  int32_t *reset = out->dev_status;
  const uint16_t *y = h;
  if (p.d_ff > 0) {
    uint16_t *ybuf = out->hidden ? out->hidden : at<uint16_t>(ws, p.o_y);
    SV_CHECK(run_mlp(p, w, h, p.M_t, nullptr, ybuf, ws, reset, st));
    reset = nullptr;
    y = ybuf;
  }
  float *logits = out->logits ? out->logits : (greedy ? nullptr : at<float>(ws, p.o_logits));
  GemmArgs g = base_args();
  g.x1 = y; g.ldx1 = p.d; g.m1 = p.M_t; g.x2 = (!greedy && K > 0) ? h_draft : y; g.ldx2 = p.d;
  g.M = p.M_lm; g.N = p.V; g.K = p.d; set_lm(g, w);
  g.logits = logits; g.ldl = p.V;
  g.parts = at<StatPart>(ws, p.o_parts); g.nslots = p.lm.nslots;
  g.invT = invT; g.want_s = (!greedy || out->diag) ? 1 : 0;
  g.status_reset = reset;
  int32_t *sync = at<int32_t>(ws, p.o_sync);
  g.counter_reset = sync;  // [0] the call's arrival counter, [1 + b] request b's block meetings
  g.counter_reset_n = greedy ? 1 : 1 + B;
  SV_CHECK(run_gemm_timed(p.lm, g, EPI_LOGITS, out, st));
  TreeArgs a = {};
  a.B = B; a.K = K; a.V = p.V; a.invT = invT; a.greedy = greedy ? 1 : 0;
  a.parts_t = g.parts; a.nslots_t = p.lm.nslots;
  a.parts_d = g.parts + (size_t)p.M_t * p.lm.nslots; a.nslots_d = p.lm.nslots;
  a.logits_t = logits; a.logits_d = logits ? logits + (size_t)p.M_t * p.V : nullptr;
  a.tokens = tokens; a.parent = parent; a.u = u;
  a.accepted_len = out->accepted_len; a.emitted = out->emitted; a.path = path;
  a.dev_status = out->dev_status; a.diag = out->diag;
  a.done_cnt = sync;
  a.fin = FinalizeArgs{out->accepted_len, nullptr, B, K, out->tau, out->counters};
  if (!greedy) {
    a.chunk_sums = at<float>(ws, p.o_tree);
    a.partials = a.chunk_sums + (size_t)B * tree_chunks(p.V);
    a.meet = sync + 1;
    // a block waits for the others at most wait_polls polls per meeting (default 65,536,
    // about 65 ms); 0 makes every meeting time out
    a.spin_limit = wait_polls < 0 ? 1 << 16 : wait_polls;
  }
  SV_CHECK(launch_tree(a, st));
  return SV_OK;
}

SV_API int spec_commit(const sv_cache *c, const int32_t *accepted_len, const int32_t *verify_len,
                       const int32_t *path, int B, int Kmax, int32_t *dev_status, void *stream) {
  if (!c || !accepted_len || !c->seq_len || B < 1 || Kmax < 0 || Kmax > 63) return SV_EINVAL;
  if (c->n_layers < 0 || c->rec_bytes < 0 || c->rec_bytes % 16 != 0) return SV_EINVAL;
  if (c->n_layers > 0) {
    if (!c->kv || !aligned16(c->kv) || !c->block_table || c->block_size < 1 || c->max_blocks < 1 ||
        c->n_blocks < 1 || c->entry_bytes < 16 || c->entry_bytes % 16 != 0 || c->layer_stride < 0 ||
        c->half_stride < 0 || c->layer_stride % 16 != 0 || c->half_stride % 16 != 0)
      return SV_EINVAL;
  }
  if (c->rec_bytes > 0 &&
      (!c->rec_state || !c->rec_snap || !aligned16(c->rec_state) || !aligned16(c->rec_snap)))
    return SV_EINVAL;
  CommitArgs a{};
  a.kv = static_cast<uint8_t *>(c->kv);
  a.layer_stride = c->layer_stride;
  a.half_stride = c->half_stride;
  a.n_layers = c->n_layers;
  a.block_size = c->block_size;
  a.entry_bytes = c->entry_bytes;
  a.max_blocks = c->max_blocks;
  a.n_blocks = c->n_blocks;
  a.block_table = c->block_table;
  a.seq_len = c->seq_len;
  a.rec_state = static_cast<uint8_t *>(c->rec_state);
  a.rec_snap = static_cast<const uint8_t *>(c->rec_snap);
  a.rec_bytes = c->rec_bytes;
  a.accepted_len = accepted_len;
  a.verify_len = verify_len;
  a.path = path;
  a.B = B;
  a.Kmax = Kmax;
  a.dev_status = dev_status;
  SV_CHECK(launch_commit(a, static_cast<hipStream_t>(stream)));
  return SV_OK;
}

SV_API const char *sv_last_hip_error(void) { return g_last_hip_error; }

SV_API const char *sv_version(void) { return "specverify 0.1.0 (gfx950)"; }

SV_API const char *sv_strerror(int code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_EWORKSPACE: return "workspace too small";
    case SV_EHIP: return "HIP runtime error";
    case SV_ESCRATCH: return "sizes need more workspace than the library's static scratch holds";
    default: return "unknown error";
  }
}
