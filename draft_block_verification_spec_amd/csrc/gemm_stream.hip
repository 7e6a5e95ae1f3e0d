// Weight-streaming GEMM for few rows (M <= 32): out[m, n] = sum_k X[m, k] W[n, k].
//
// At small batch the verification pass is bound by reading the weights once
// (Wildberries page, "Where speculative decoding came from": scoring eight
// positions costs about as much as one because the weights are read once).  This
// kernel therefore streams W exactly once from HBM with 16-byte loads and keeps
// the few activation rows resident in registers:
//
//  * one persistent 512-thread workgroup per CU owns a contiguous range of 16-row
//    tiles of W;
//  * the 8 waves split the reduction: wave w covers 16 MFMA k-steps (512 values)
//    of every 4096-wide chunk of K, so each wave keeps its slice of X (the MFMA A
//    operand, 16 rows per block) in VGPRs for the whole sweep when K <= 4096;
//  * W tiles feed the B operand of v_mfma_f32_16x16x32_bf16.  HBM streams fastest
//    when every row is read in runs of 256 bytes or more, while the MFMA wants each
//    lane on its own row (16 rows x 64 bytes per load).  So when K is a whole number
//    of 4096-value chunks each wave load reads 4 rows x 256 contiguous bytes, and a
//    private 4 KiB LDS slot per wave turns 4 such loads (16 rows x 128 values) into
//    the fragments of 4 k-steps: one 128-bit LDS write and one read per lane and
//    load, XOR-swizzled so both are free of bank conflicts, no barriers.  Each of
//    the 16 loads of a step is re-issued for the next step as soon as its data is in
//    LDS, so about 16 KiB per wave stay in flight;
//  * the 8 partial accumulators of a tile are summed in a fixed order through LDS
//    (deterministic), then the epilogue runs: fp32 logits + running per-row
//    statistics, SwiGLU with paired gate/up rows, or residual add, bf16 output.
#include <atomic>
#include <type_traits>

#include "sv_device.h"

namespace sv {

namespace {

constexpr int STEPS = 16;     // MFMA k-steps (32 values) per wave per chunk
constexpr int WAVES = 8;
constexpr int CHUNK_KS = STEPS * WAVES;  // k-steps per chunk (4096 values)
constexpr int F8_MAX_COLS = 2048;        // FP8: columns of one workgroup whose scales are staged

// KM (K mode): 1 = K is one 4096-value chunk, 2 = K is several whole chunks, 0 = any
// other K.  With whole chunks (FULL) every wave owns exactly STEPS
// k-steps of every chunk and the hot loop has no data-dependent control flow:
// every load is issued unconditionally from a valid (clamped) address, which lets
// the compiler keep the 16 loads of a step in flight with partial vmcnt waits.
// Rows beyond M read a clamped row and their results are dropped; weight rows
// beyond N likewise.  The general path masks the tail of K with zero operands.
template <int MB, int EPI, int KM, bool F8>
__global__ __launch_bounds__(512) void k_stream(const GemmArgs a) {
  constexpr bool FULL = KM != 0;
  constexpr bool RELOAD_A = KM != 1;  // activations change with the chunk
  constexpr bool PAIR = (EPI == EPI_SWIGLU);
  constexpr int NACC = PAIR ? 2 * MB : MB;
  constexpr int NW = PAIR ? 2 : 1;  // weight streams
  // FP8 weights: one byte per value, so a 256-byte run of a row holds 8 k-steps and a
  // step of 16 k-steps needs 8 loads (16 with bf16); the general path reads 8 bytes
  // per lane and k-step.
  constexpr int ES = F8 ? 1 : 2;                // bytes per weight value
  constexpr int WL = (F8 && FULL) ? 8 : STEPS;  // weight loads per wave and step
  constexpr int GK = F8 ? 8 : 4;                // k-steps per reshaping group
  using WT = typename std::conditional<F8 && !FULL, u32x2, u32x4>::type;
  // Every weight byte is read exactly once per call: nontemporal loads (measured
  // faster for all three GEMMs of the step).
  auto ldw = [](const uint8_t *p) -> WT { return __builtin_nontemporal_load(reinterpret_cast<const WT *>(p)); };
  __shared__ float red[2][WAVES * NACC * 4 * 64];
  // per-wave reshaping slots (whole-chunk K only): [wave][stream][16 rows x 256 bytes]
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[FULL ? WAVES * NW * 4096 : 16];
  // FP8: the row scales of the workgroup's column range, staged once
  __shared__ float sscale[F8 ? NW * F8_MAX_COLS : 1];
  // Outputs of the workgroup's whole column range are kept in LDS and written once at
  // the end (when a.buf_cols > 0): stores inside the streaming loop would share the
  // vector-memory counter with the weight loads and stall them.
  extern __shared__ float obuf[];

  if (a.status_reset && blockIdx.x == 0 && threadIdx.x == 0) *a.status_reset = 0;
  if (a.counter_reset && blockIdx.x == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < max(1, a.counter_reset_n); i += blockDim.x) a.counter_reset[i] = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = live_rows(a);
  if (M < 0) return;  // another launch of the same product does the work
  if (a.nslots_out && blockIdx.x == 0 && threadIdx.x == 0) *a.nslots_out = a.nslots_plan;
  const int N = a.N;
  const int nks = a.K >> 5;
  const int nch = (nks + CHUNK_KS - 1) / CHUNK_KS;
  // The workgroup's columns [c_begin, c_end) split N in groups of 4 columns, so that no
  // workgroup streams more than a sixteenth of a tile beyond its share: its last tile
  // may be partial, and its missing rows repeat the last valid row's addresses, which
  // the memory pipeline merges (no extra HBM bytes).
  const int G = gridDim.x, g = blockIdx.x;
  const int nq = (N + 3) >> 2;
  const int c_begin = min(N, 4 * (int)((long)g * nq / G));
  const int c_end = min(N, 4 * (int)((long)(g + 1) * nq / G));
  const int nsteps = ((c_end - c_begin + 15) >> 4) * nch;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const long K = a.K;

  auto xrow = [&](int m) -> const uint16_t * {
    m = min(m, max(M, 1) - 1);
    return m < a.m1 ? a.x1 + (long)m * a.ldx1 : a.x2 + (long)(m - a.m1) * a.ldx2;
  };

  bf16x8 A[MB][STEPS];
  WT Wr[WL];
  WT Ur[PAIR ? WL : 1];
  const bf16x8 zero8 = {};
  const uint8_t *wb = reinterpret_cast<const uint8_t *>(a.w);
  const uint8_t *wb2 = reinterpret_cast<const uint8_t *>(a.w2);

  auto kstep = [&](int chunk, int s) { return chunk * CHUNK_KS + wave * STEPS + s; };
  auto load_a = [&](int chunk, int s, int mb) -> bf16x8 {
    const int ks = kstep(chunk, s);
    if constexpr (FULL) {
      return as_bf16x8(ld16(xrow(mb * 16 + r16) + ks * 32 + kq));
    } else {
      if (ks < nks) return as_bf16x8(ld16(xrow(mb * 16 + r16) + ks * 32 + kq));
      return zero8;
    }
  };
  // Weight load s of a step.  Whole chunks: group g holds GK k-steps (a 256-byte run of
  // every row, 128 bf16 or 256 FP8 values) of the wave's 512 values; load s%4 of the
  // group covers rows 4 (s%4) + l/16, 16 bytes at 16 (l%16) of the run.  General K: the
  // MFMA layout straight from memory (row l%16, 8 values at 8 (l/16)).
  auto wptr = [&](const uint8_t *base, int tile, int chunk, int s) -> const uint8_t * {
    if constexpr (FULL) {
      const int n = min(c_begin + tile * 16 + 4 * (s & 3) + (lane >> 4), c_end - 1);
      return base + ((long)n * K + chunk * (CHUNK_KS * 32) + wave * (STEPS * 32)) * ES + (s >> 2) * 256 + r16 * 16;
    } else {
      const int ks = min(kstep(chunk, s), nks - 1);
      const int n = min(c_begin + tile * 16 + r16, c_end - 1);
      return base + ((long)n * K + ks * 32 + kq) * ES;
    }
  };
  // 8 FP8 values (one per byte, in order) to the bf16 MFMA operand (exact).
  auto f8_bf16 = [](u32x2 v) -> bf16x8 {
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true));
    return as_bf16x8(r);
  };
  // B operand of a general-path load
  auto wop = [&](const WT &v) -> bf16x8 {
    if constexpr (F8 && !FULL) return f8_bf16(v);
    else return as_bf16x8(v);
  };
  // LDS reshaping (whole chunks): row r's 16-byte chunk c of a group sits at chunk c ^ r.
  uint8_t *tw = tbuf + (FULL ? wave * NW * 4096 : 0);
  auto put4 = [&](uint8_t *slot, int i, const u32x4 &v) {  // load i of a group, this lane's 16 bytes
    const int r = 4 * i + (lane >> 4);
    *reinterpret_cast<u32x4 *>(slot + r * 256 + ((r16 ^ r) << 4)) = v;
  };
  auto frag = [&](const uint8_t *slot, int j) -> bf16x8 {  // B operand of k-step j of a group
    if constexpr (F8) {
      const int q = lane >> 4;  // 8 bytes at 32 j + 8 q of row r16
      return f8_bf16(*reinterpret_cast<const u32x2 *>(slot + r16 * 256 + ((((2 * j) + (q >> 1)) ^ r16) << 4) +
                                                      (q & 1) * 8));
    } else {
      return *reinterpret_cast<const bf16x8 *>(slot + r16 * 256 + ((((4 * j) + (lane >> 4)) ^ r16) << 4));
    }
  };

  // statistics of the row this thread reduces (EPI_LOGITS)
  StatPart st = stat_empty();
  const int e = threadIdx.x;                 // element handled in the epilogue
  const bool has_elem = e < MB * 256;
  const int e_mb = e >> 8, e_r = (e >> 6) & 3, e_ln = e & 63;
  const int e_m = e_mb * 16 + 4 * (e_ln >> 4) + e_r;
  const int e_n16 = e_ln & 15;

  if constexpr (F8) {
    // row scales of this workgroup's columns (the launcher checks they fit)
    const int n0 = c_begin, cols = c_end - c_begin;
    for (int i = threadIdx.x; i < cols; i += blockDim.x) {
      sscale[i] = a.wscale[n0 + i];
      if constexpr (PAIR) sscale[F8_MAX_COLS + i] = a.wscale2[n0 + i];
    }
  }
  // First step's operands.  The loads are issued in exactly the order in which the loop
  // refills them (pinned with sched_barrier): the wait counts at the top of the loop are
  // merged over the loop entry and the back edge, so any other order makes every step
  // wait for most of its loads before the first refill, emptying the pipeline.
  if (nsteps > 0) {
    if constexpr (!RELOAD_A) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) A[mb][s] = load_a(0, s, mb);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (FULL) {
#pragma unroll
      for (int g = 0; g < STEPS / GK; ++g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Wr[4 * g + i] = ldw(wptr(wb, 0, 0, 4 * g + i));
          if constexpr (PAIR) Ur[4 * g + i] = ldw(wptr(wb2, 0, 0, 4 * g + i));
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (RELOAD_A) {
#pragma unroll
          for (int j = 0; j < GK; ++j) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) A[mb][GK * g + j] = load_a(0, GK * g + j, mb);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        Wr[s] = ldw(wptr(wb, 0, 0, s));
        if constexpr (PAIR) Ur[s] = ldw(wptr(wb2, 0, 0, s));
        if constexpr (RELOAD_A) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) A[mb][s] = load_a(0, s, mb);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  f32x4 acc[NACC];
  int parity = 0;
  // One step: the MFMAs of the current operands, each slot refilled right after use
  // with the next step's operands.  The last step is peeled (PF = false) so it issues
  // no prefetch at all and the loop body stays free of branches around loads.
  auto mma_step = [&](int stp, auto pf) {
    constexpr bool PF = decltype(pf)::value;
    const int c = stp % nch;
    const int nstp = stp + 1;
    const int ntile = nstp / nch, nc = nstp % nch;  // tile index within the workgroup
    if (c == 0) {
#pragma unroll
      for (int q = 0; q < NACC; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (FULL) {
#pragma unroll
      for (int g = 0; g < STEPS / GK; ++g) {
        // the group's 4 loads (per stream) into this wave's slot, then refill them
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          put4(tw, i, Wr[4 * g + i]);
          if constexpr (PAIR) put4(tw + 4096, i, Ur[4 * g + i]);
        }
        if constexpr (PF) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            Wr[4 * g + i] = ldw(wptr(wb, ntile, nc, 4 * g + i));
            if constexpr (PAIR) Ur[4 * g + i] = ldw(wptr(wb2, ntile, nc, 4 * g + i));
          }
        }
#pragma unroll
        for (int j = 0; j < GK; ++j) {
          const int ks = GK * g + j;
          const bf16x8 bw = frag(tw, j);
          bf16x8 bu = bw;
          if constexpr (PAIR) bu = frag(tw + 4096, j);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            if constexpr (PAIR) {
              acc[2 * mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][ks], bw, acc[2 * mb], 0, 0, 0);
              acc[2 * mb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][ks], bu, acc[2 * mb + 1], 0, 0, 0);
            } else {
              acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][ks], bw, acc[mb], 0, 0, 0);
            }
          }
          if constexpr (PF && RELOAD_A) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) A[mb][ks] = load_a(nc, ks, mb);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (PAIR) {
          acc[2 * mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][s], wop(Wr[s]), acc[2 * mb], 0, 0, 0);
          acc[2 * mb + 1] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][s], wop(Ur[s]), acc[2 * mb + 1], 0, 0, 0);
        } else {
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][s], wop(Wr[s]), acc[mb], 0, 0, 0);
        }
      }
      if constexpr (PF) {
        Wr[s] = ldw(wptr(wb, ntile, nc, s));
        if constexpr (PAIR) Ur[s] = ldw(wptr(wb2, ntile, nc, s));
        if constexpr (RELOAD_A) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) A[mb][s] = load_a(nc, s, mb);
        }
      }
      // keep "use slot s, refill slot s" in program order so loads stay spread over the step
      __builtin_amdgcn_sched_barrier(0);
    }
    }
  };
  for (int stp = 0; stp < nsteps; ++stp) {
    const int tile = stp / nch, c = stp % nch;
    if (stp + 1 < nsteps) mma_step(stp, std::true_type{});
    else mma_step(stp, std::false_type{});
    if (c != nch - 1) continue;

    // ---- deterministic cross-wave reduction of the tile through LDS
    float *rb = red[parity];
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) rb[((wave * NACC + q) * 4 + r) * 64 + lane] = acc[q][r];
    __syncthreads();
    if (has_elem) {
      const int n = c_begin + tile * 16 + e_n16;
      const int m = e_m;
      float v0 = 0.f, v1 = 0.f;
      const int q0 = PAIR ? 2 * e_mb : e_mb;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        v0 += rb[((w * NACC + q0) * 4 + e_r) * 64 + e_ln];
        if constexpr (PAIR) v1 += rb[((w * NACC + q0 + 1) * 4 + e_r) * 64 + e_ln];
      }
      if (m < M && n < c_end) {
        const int bc = n - c_begin;  // column within the workgroup's range
        if constexpr (F8) {
          v0 *= sscale[bc];
          if constexpr (PAIR) v1 *= sscale[F8_MAX_COLS + bc];
        }
        if constexpr (EPI == EPI_LOGITS) {
          if (a.logits) {
            if (a.buf_cols) obuf[m * a.buf_cols + bc] = v0;
            else a.logits[(long)m * a.ldl + n] = v0;
          }
          stat_push(st, v0, n, a.invT, a.want_s != 0);
        } else {
          uint16_t o;
          if constexpr (EPI == EPI_SWIGLU) {
            const float sg = v0 / (1.f + __expf(-v0));
            o = f32_to_bf16(sg * v1);
          } else {
            const float hv = bf16_to_f32(a.resid[(long)m * a.ldr + n]);
            o = f32_to_bf16(hv + v0);
          }
          if (a.buf_cols) reinterpret_cast<uint16_t *>(obuf)[m * a.buf_cols + bc] = o;
          else a.out[(long)m * a.ldo + n] = o;
        }
      }
    }
    parity ^= 1;
  }

  if constexpr (EPI == EPI_LOGITS) {
    // 16 consecutive threads share a row: butterfly over them, one writes the partial.
    const bool ws = a.want_s != 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      StatPart o = stat_shfl_xor(st, off);
      st = stat_merge(st, o, a.invT, ws);
    }
    if (has_elem && e_n16 == 0 && e_m < M) a.parts[(long)e_m * a.nslots + g] = st;
  }
  // flush the buffered outputs: each row's column range is contiguous in memory
  if (a.buf_cols && nsteps > 0 && (EPI != EPI_LOGITS || a.logits)) {
    __syncthreads();
    const int cols = c_end - c_begin;
    const int n0 = c_begin;
    const int rows = min(M, MB * 16);
    // one wave per row; 16-byte stores when every row start is 16-byte aligned (the
    // buffer rows are: buf_cols is a multiple of 16 values)
    if constexpr (EPI == EPI_LOGITS) {
      const bool vec = (a.ldl & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0;
      for (int m = wave; m < rows; m += WAVES) {
        float *dst = a.logits + (long)m * a.ldl + n0;
        const float *src = obuf + m * a.buf_cols;
        if (vec) {
          for (int c = lane * 4; c < cols; c += 256) {
            if (c + 4 <= cols) *reinterpret_cast<f32x4 *>(dst + c) = *reinterpret_cast<const f32x4 *>(src + c);
            else
              for (int i = c; i < cols; ++i) dst[i] = src[i];
          }
        } else {
          for (int c = lane; c < cols; c += 64) dst[c] = src[c];
        }
      }
    } else {
      for (int m = wave; m < rows; m += WAVES) {
        uint16_t *dst = a.out + (long)m * a.ldo + n0;
        const uint16_t *src = reinterpret_cast<const uint16_t *>(obuf) + m * a.buf_cols;
        for (int c = lane; c < cols; c += 64) dst[c] = src[c];
      }
    }
  }
}

}  // namespace

bool stream_ok(int M, int epi) { return M >= 1 && (epi == EPI_SWIGLU ? M <= 16 : M <= 32); }

int stream_grid(const GemmArgs &a, int epi) {
  (void)epi;
  const int ntiles = (a.N + 15) / 16;
  return ntiles < num_cus() ? ntiles : num_cus();
}

// Output buffer per workgroup: up to 32 rows x its column range (fp32 logits or bf16),
// in the LDS left over by the kernel's static buffers (160 KiB per workgroup on gfx950).
constexpr size_t LDS_PER_CU = 160 * 1024;
constexpr size_t OBUF_MAX = 96 * 1024;

template <int MB, int EPI, int KM, bool F8>
constexpr size_t stream_static_lds() {
  constexpr size_t nacc = EPI == EPI_SWIGLU ? 2 * MB : MB;
  constexpr size_t nw = EPI == EPI_SWIGLU ? 2 : 1;
  constexpr size_t red = 2 * WAVES * nacc * 4 * 64 * sizeof(float);
  constexpr size_t tb = KM != 0 ? (size_t)WAVES * nw * 4096 : 16;
  constexpr size_t sc = F8 ? nw * F8_MAX_COLS * sizeof(float) : sizeof(float);
  return red + tb + sc;
}

template <int MB, int EPI, int KM, bool F8>
hipError_t launch_one(GemmArgs a, int grid, hipStream_t st) {
  constexpr size_t stat = stream_static_lds<MB, EPI, KM, F8>();
  constexpr size_t dyn_max = LDS_PER_CU - stat < OBUF_MAX ? LDS_PER_CU - stat : OBUF_MAX;
  // columns of the widest workgroup (groups of 4), rounded up to whole tiles
  const int nq = (a.N + 3) / 4;
  const int cols = 16 * ((4 * ((nq + grid - 1) / grid) + 15) / 16);
  if (F8 && cols > F8_MAX_COLS) return hipErrorInvalidValue;
  const size_t esz = EPI == EPI_LOGITS ? 4 : 2;
  size_t shm = (size_t)MB * 16 * cols * esz;
  a.buf_cols = 0;
  if (shm <= dyn_max && (EPI != EPI_LOGITS || a.logits)) {
    a.buf_cols = cols;
    // the attribute belongs to the current device: set once per device and instantiation
    static std::atomic<unsigned long long> attr_set{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = 1ull << (dev & 63);
    if (!(attr_set.load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_stream<MB, EPI, KM, F8>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_max);
      if (e != hipSuccess) return e;
      attr_set.fetch_or(bit, std::memory_order_release);
    }
  } else {
    shm = 0;
  }
  hipLaunchKernelGGL((k_stream<MB, EPI, KM, F8>), dim3(grid), dim3(512), shm, st, a);
  return hipGetLastError();
}

template <int KM, bool F8>
hipError_t launch_stream_t(const GemmArgs &a, int epi, int grid, hipStream_t st) {
  const bool two = a.M > 16;
  switch (epi) {
    case EPI_LOGITS:
      return two ? launch_one<2, EPI_LOGITS, KM, F8>(a, grid, st) : launch_one<1, EPI_LOGITS, KM, F8>(a, grid, st);
    case EPI_SWIGLU:
      return launch_one<1, EPI_SWIGLU, KM, F8>(a, grid, st);
    case EPI_RESID:
      return two ? launch_one<2, EPI_RESID, KM, F8>(a, grid, st) : launch_one<1, EPI_RESID, KM, F8>(a, grid, st);
    default:
      return hipErrorInvalidValue;
  }
}

template <bool F8>
hipError_t launch_stream_q(const GemmArgs &a, int epi, int grid, hipStream_t st) {
  if (a.K == CHUNK_KS * 32) return launch_stream_t<1, F8>(a, epi, grid, st);
  if (a.K % (CHUNK_KS * 32) == 0) return launch_stream_t<2, F8>(a, epi, grid, st);
  return launch_stream_t<0, F8>(a, epi, grid, st);
}

hipError_t launch_gemm_stream(const GemmArgs &a, int epi, int grid, hipStream_t st) {
  if (a.wfp8) {
    if (!a.wscale || (epi == EPI_SWIGLU && !a.wscale2)) return hipErrorInvalidValue;
    return launch_stream_q<true>(a, epi, grid, st);
  }
  return launch_stream_q<false>(a, epi, grid, st);
}

}  // namespace sv
