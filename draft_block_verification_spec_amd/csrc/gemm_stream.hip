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
//  * W tiles feed the B operand of v_mfma_f32_16x16x32_bf16 straight from global
//    memory (lane l reads row l%16, 8 consecutive k at 8*(l/16)); each of the 16
//    loads of a step is re-issued for the next step as soon as its MFMA has been
//    issued, so about 16 KiB per wave stay in flight;
//  * the 8 partial accumulators of a tile are summed in a fixed order through LDS
//    (deterministic), then the epilogue runs: fp32 logits + running per-row
//    statistics, SwiGLU with paired gate/up rows, or residual add, bf16 output.
#include "sv_device.h"

namespace sv {

namespace {

constexpr int STEPS = 16;     // MFMA k-steps (32 values) per wave per chunk
constexpr int WAVES = 8;
constexpr int CHUNK_KS = STEPS * WAVES;  // k-steps per chunk (4096 values)

template <int MB, int EPI>
__global__ __launch_bounds__(512) void k_stream(const GemmArgs a) {
  constexpr bool PAIR = (EPI == EPI_SWIGLU);
  constexpr int NACC = PAIR ? 2 * MB : MB;
  __shared__ float red[2][WAVES * NACC * 4 * 64];

  if (a.status_reset && blockIdx.x == 0 && threadIdx.x == 0) *a.status_reset = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = a.M_dev ? min(a.M, *a.M_dev) : a.M;
  const int N = a.N;
  const int nks = a.K >> 5;
  const int nch = (nks + CHUNK_KS - 1) / CHUNK_KS;
  const int ntiles = (N + 15) >> 4;
  const int G = gridDim.x, g = blockIdx.x;
  const int t_begin = (int)((long)g * ntiles / G);
  const int t_end = (int)((long)(g + 1) * ntiles / G);
  const int nsteps = (t_end - t_begin) * nch;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const long K = a.K;

  auto xrow = [&](int m) -> const uint16_t * {
    return m < a.m1 ? a.x1 + (long)m * a.ldx1 : a.x2 + (long)(m - a.m1) * a.ldx2;
  };

  bf16x8 A[MB][STEPS];
  bf16x8 Wr[STEPS];
  bf16x8 Ur[PAIR ? STEPS : 1];
  const bf16x8 zero8 = {};

  auto load_a = [&](int chunk, int s, int mb) -> bf16x8 {
    const int ks = chunk * CHUNK_KS + wave * STEPS + s;
    const int m = mb * 16 + r16;
    if (ks < nks && m < M) return as_bf16x8(ld16(xrow(m) + ks * 32 + kq));
    return zero8;
  };
  auto wptr = [&](const uint16_t *base, int tile, int chunk, int s) -> const uint16_t * {
    const int ks = chunk * CHUNK_KS + wave * STEPS + s;
    const int n = min(tile * 16 + r16, N - 1);
    return base + (long)n * K + ks * 32 + kq;
  };
  auto kvalid = [&](int chunk, int s) { return chunk * CHUNK_KS + wave * STEPS + s < nks; };

  // statistics of the row this thread reduces (EPI_LOGITS)
  StatPart st = stat_empty();
  const int e = threadIdx.x;                 // element handled in the epilogue
  const bool has_elem = e < MB * 256;
  const int e_mb = e >> 8, e_r = (e >> 6) & 3, e_ln = e & 63;
  const int e_m = e_mb * 16 + 4 * (e_ln >> 4) + e_r;
  const int e_n16 = e_ln & 15;

  if (nsteps > 0) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) A[mb][s] = load_a(0, s, mb);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const bool kv = kvalid(0, s);
      Wr[s] = kv ? as_bf16x8(ld_nt(wptr(a.w, t_begin, 0, s))) : zero8;
      if constexpr (PAIR) Ur[s] = kv ? as_bf16x8(ld_nt(wptr(a.w2, t_begin, 0, s))) : zero8;
    }
  }

  f32x4 acc[NACC];
  int parity = 0;
  for (int stp = 0; stp < nsteps; ++stp) {
    const int tile = t_begin + stp / nch, c = stp % nch;
    const int nstp = stp + 1;
    const bool has_next = nstp < nsteps;
    const int ntile = t_begin + nstp / nch, nc = nstp % nch;
    if (c == 0) {
#pragma unroll
      for (int q = 0; q < NACC; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (PAIR) {
          acc[2 * mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][s], Wr[s], acc[2 * mb], 0, 0, 0);
          acc[2 * mb + 1] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][s], Ur[s], acc[2 * mb + 1], 0, 0, 0);
        } else {
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][s], Wr[s], acc[mb], 0, 0, 0);
        }
      }
      if (has_next) {
        const bool kv = kvalid(nc, s);
        Wr[s] = kv ? as_bf16x8(ld_nt(wptr(a.w, ntile, nc, s))) : zero8;
        if constexpr (PAIR) Ur[s] = kv ? as_bf16x8(ld_nt(wptr(a.w2, ntile, nc, s))) : zero8;
        if (nch > 1) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) A[mb][s] = load_a(nc, s, mb);
        }
      }
    }
    if (c != nch - 1) continue;

    // ---- deterministic cross-wave reduction of the tile through LDS
    float *rb = red[parity];
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) rb[((wave * NACC + q) * 4 + r) * 64 + lane] = acc[q][r];
    __syncthreads();
    if (has_elem) {
      const int n = tile * 16 + e_n16;
      const int m = e_m;
      float v0 = 0.f, v1 = 0.f;
      const int q0 = PAIR ? 2 * e_mb : e_mb;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        v0 += rb[((w * NACC + q0) * 4 + e_r) * 64 + e_ln];
        if constexpr (PAIR) v1 += rb[((w * NACC + q0 + 1) * 4 + e_r) * 64 + e_ln];
      }
      if (m < M && n < N) {
        if constexpr (EPI == EPI_LOGITS) {
          if (a.logits) a.logits[(long)m * a.ldl + n] = v0;
          stat_push(st, v0, n, a.invT, a.want_s != 0);
        } else if constexpr (EPI == EPI_SWIGLU) {
          const float sg = v0 / (1.f + __expf(-v0));
          a.out[(long)m * a.ldo + n] = f32_to_bf16(sg * v1);
        } else if constexpr (EPI == EPI_RESID) {
          const float hv = bf16_to_f32(a.resid[(long)m * a.ldr + n]);
          a.out[(long)m * a.ldo + n] = f32_to_bf16(hv + v0);
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
}

}  // namespace

bool stream_ok(int M, int epi) { return M >= 1 && (epi == EPI_SWIGLU ? M <= 16 : M <= 32); }

int stream_grid(const GemmArgs &a, int epi) {
  (void)epi;
  const int ntiles = (a.N + 15) / 16;
  return ntiles < num_cus() ? ntiles : num_cus();
}

hipError_t launch_gemm_stream(const GemmArgs &a, int epi, int grid, hipStream_t st) {
  const bool two = a.M > 16;
  dim3 blk(512), grd(grid);
  switch (epi) {
    case EPI_LOGITS:
      if (two) hipLaunchKernelGGL((k_stream<2, EPI_LOGITS>), grd, blk, 0, st, a);
      else hipLaunchKernelGGL((k_stream<1, EPI_LOGITS>), grd, blk, 0, st, a);
      break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL((k_stream<1, EPI_SWIGLU>), grd, blk, 0, st, a);
      break;
    case EPI_RESID:
      if (two) hipLaunchKernelGGL((k_stream<2, EPI_RESID>), grd, blk, 0, st, a);
      else hipLaunchKernelGGL((k_stream<1, EPI_RESID>), grd, blk, 0, st, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sv
