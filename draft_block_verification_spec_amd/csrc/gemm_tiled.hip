// LDS-tiled MFMA GEMM for larger row counts: out[m, n] = sum_k X[m, k] W[n, k].
//
// Once B*(K+1) rows share each weight read the verification pass stops being
// bound by HBM and becomes compute-bound (Wildberries page, "A bit of theory",
// Statement 3: under load the step time grows with B*(K+1)).  This kernel tiles
// BM x BN outputs per 256-thread workgroup (2 x 2 waves), stages 64-wide k slices
// of both operands through double-buffered LDS (rows padded by 16 bytes so the
// 128-bit operand reads are bank-conflict free) and issues
// v_mfma_f32_32x32x16_bf16 on 32x32 blocks.  Workgroups are mapped XCD-major so
// the row tiles that share a weight tile run on one XCD and share its L2.
// Split-K writes fp32 partials that a second kernel reduces in a fixed order.
#include "sv_device.h"

namespace sv {

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;

// PAIR: the weight rows of a tile are [32 gate | 32 up] groups of the same outputs.
template <int BM, int BN, int EPI, bool PAIR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_tiled(const GemmArgs a) {
  constexpr int WTM = BM / 2, WTN = BN / 2, TM = WTM / 32, TN = WTN / 32;
  constexpr int ACH = BM * 8 / 256, BCH = BN * 8 / 256;
  static_assert(ACH >= 1 && BCH >= 1, "tile too small");
  static_assert(!PAIR || (WTN % 64) == 0, "paired tiles need gate/up block pairs");
  // operand tiles, double-buffered; reused by the statistics epilogue after the main loop
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * LDK];
  uint16_t(*As)[BM * LDK] = reinterpret_cast<uint16_t(*)[BM * LDK]>(smem);
  uint16_t(*Bs)[BN * LDK] = reinterpret_cast<uint16_t(*)[BN * LDK]>(smem + 2 * BM * LDK);

  if (a.status_reset && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) *a.status_reset = 0;
  if (a.counter_reset && blockIdx.x == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < max(1, a.counter_reset_n); i += blockDim.x) a.counter_reset[i] = 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int M = a.M;
  if (a.M_dev) M = min(M, *a.M_dev);
  const int Ncols = PAIR ? 2 * a.N : a.N;  // columns of the weight-row space
  const int tiles_m = (a.M + BM - 1) / BM;
  const int G = gridDim.x;
  int lin = blockIdx.x;
  if ((G & 7) == 0) lin = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int tmi = lin % tiles_m, tni = lin / tiles_m;
  const int m0 = tmi * BM, n0 = tni * BN;
  if (m0 >= M) return;

  const int splits = gridDim.z, z = blockIdx.z;
  const int nkt_total = a.K / BK;
  const int per = (nkt_total + splits - 1) / splits;
  const int kt0 = z * per;
  const int kt1 = min(nkt_total, kt0 + per);
  const int nkt = kt1 > kt0 ? kt1 - kt0 : 0;

  // ---- global -> register staging.  Rows past M (or N) read a clamped valid row;
  // their results are never stored, and the loads stay free of branches.
  const uint16_t *arow[ACH];
  const uint16_t *brow[BCH];
  const int mlast = max(M, 1) - 1;
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int q = tid + i * 256, r = q >> 3;
    const int m = min(m0 + r, mlast);
    arow[i] = (m < a.m1 ? a.x1 + (long)m * a.ldx1 : a.x2 + (long)(m - a.m1) * a.ldx2) + (q & 7) * 8;
  }
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int q = tid + i * 256, r = q >> 3;
    if constexpr (PAIR) {
      // tile columns: 64-wide groups of [32 gate rows | 32 up rows] of the same outputs
      const int p = r >> 6, half = (r >> 5) & 1, rr = r & 31;
      const int n = min((n0 >> 1) + p * 32 + rr, a.N - 1);
      brow[i] = (half ? a.w2 : a.w) + (long)n * a.K + (q & 7) * 8;
    } else {
      const int n = min(n0 + r, a.N - 1);
      brow[i] = a.w + (long)n * a.K + (q & 7) * 8;
    }
  }
  u32x4 ra[ACH], rb[BCH];
  auto gload = [&](int kt) {
    const long ko = (long)kt * BK;
#pragma unroll
    for (int i = 0; i < ACH; ++i) ra[i] = ld16(arow[i] + ko);
#pragma unroll
    for (int i = 0; i < BCH; ++i) rb[i] = ld_nt(brow[i] + ko);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int q = tid + i * 256;
      *reinterpret_cast<u32x4 *>(&As[buf][(q >> 3) * LDK + (q & 7) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int q = tid + i * 256;
      *reinterpret_cast<u32x4 *>(&Bs[buf][(q >> 3) * LDK + (q & 7) * 8]) = rb[i];
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nkt > 0) {
    gload(kt0);
    sstore(0);
    __syncthreads();
  }
  const int l32 = lane & 31, khalf = (lane >> 5) * 8;
  for (int t = 0; t < nkt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nkt) gload(kt0 + t + 1);
    // operand fragments are double-buffered in registers: the LDS reads of step
    // kk+1 are issued before the MFMAs of step kk
    bf16x8 af[2][TM], bfr[2][TN];
    auto lfrag = [&](int set, int kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[set][i] = *reinterpret_cast<const bf16x8 *>(&As[buf][(wm * WTM + i * 32 + l32) * LDK + kk * 16 + khalf]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[set][j] = *reinterpret_cast<const bf16x8 *>(&Bs[buf][(wn * WTN + j * 32 + l32) * LDK + kk * 16 + khalf]);
    };
    lfrag(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < BK / 16) lfrag(cur ^ 1, kk + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (t + 1 < nkt) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Lane l of block (i, j) holds column l%32 and, for register r,
  // row (r/4)*8 + (l/32)*4 + r%4 of the 32x32 block.
  const int rsub = (lane >> 5) * 4;
  if constexpr (EPI == EPI_RAW) {
    float *P = a.partial + (long)z * a.M * Ncols;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WTN + j * 32 + l32;
        if (n >= Ncols) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          if (m < M) P[(long)m * Ncols + n] = acc[i][j][r];
        }
      }
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jp = 0; jp < TN / 2; ++jp) {
        const int n = (n0 >> 1) + (wn * WTN) / 2 + jp * 32 + l32;
        if (n >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          if (m < M) {
            const float gv = acc[i][2 * jp][r], uv = acc[i][2 * jp + 1][r];
            const float sg = gv / (1.f + __expf(-gv));
            a.out[(long)m * a.ldo + n] = f32_to_bf16(sg * uv);
          }
        }
      }
  } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WTN + j * 32 + l32;
        if (n >= a.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          if (m < M) {
            const float hv = bf16_to_f32(a.resid[(long)m * a.ldr + n]);
            a.out[(long)m * a.ldo + n] = f32_to_bf16(hv + acc[i][j][r]);
          }
        }
      }
  } else {  // EPI_LOGITS
    // Logits go out straight from the accumulators (32 consecutive columns per
    // register).  For the row statistics each wave stages one 32-row group of its
    // tile in LDS at a time (row stride padded to 65 floats), then lane l scans row
    // l%32 over half l/32 of the wave's columns in increasing order and the two
    // halves are merged with one shuffle.
    const bool ws = a.want_s != 0;
    const int slot = tni * 2 + wn;
    constexpr int SROW = WTN + 1;
    static_assert(4 * 32 * SROW * 4 <= 2 * (BM + BN) * LDK * 2, "staging area too small");
    __syncthreads();
    float *stage = reinterpret_cast<float *>(smem) + wave * (32 * SROW);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WTN + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = (r >> 2) * 8 + rsub + (r & 3);
          const int m = m0 + wm * WTM + i * 32 + rr;
          stage[rr * SROW + j * 32 + l32] = acc[i][j][r];
          if (a.logits && m < M && n < a.N) a.logits[(long)m * a.ldl + n] = acc[i][j][r];
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are done
      const int rr = l32, half = lane >> 5;
      const int m = m0 + wm * WTM + i * 32 + rr;
      StatPart st = stat_empty();
      const int c0 = half * (WTN / 2);
      for (int c = 0; c < WTN / 2; ++c) {
        const int n = n0 + wn * WTN + c0 + c;
        if (n < a.N) stat_push(st, stage[rr * SROW + c0 + c], n, a.invT, ws);
      }
      st = stat_merge(st, stat_shfl_xor(st, 32), a.invT, ws);
      if (half == 0 && m < M) a.parts[(long)m * a.nslots + slot] = st;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next group
    }
  }
}

// Fixed-order reduction of split-K partials followed by the elementwise epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void k_splitk_reduce(const GemmArgs a, int splits, int bn) {
  int M = a.M;
  if (a.M_dev) M = min(M, *a.M_dev);
  const long total = (long)M * a.N;
  const int Ncols = (EPI == EPI_SWIGLU) ? 2 * a.N : a.N;
  const long stride = (long)a.M * Ncols;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < total; idx += (long)gridDim.x * blockDim.x) {
    const int m = (int)(idx / a.N), n = (int)(idx % a.N);
    if constexpr (EPI == EPI_SWIGLU) {
      const int half_bn = bn >> 1;
      const int tni = n / half_bn, rem = n % half_bn;
      const int gcol = tni * bn + (rem >> 5) * 64 + (rem & 31);
      float gv = 0.f, uv = 0.f;
      for (int s = 0; s < splits; ++s) {
        gv += a.partial[s * stride + (long)m * Ncols + gcol];
        uv += a.partial[s * stride + (long)m * Ncols + gcol + 32];
      }
      const float sg = gv / (1.f + __expf(-gv));
      a.out[(long)m * a.ldo + n] = f32_to_bf16(sg * uv);
    } else {
      float v = 0.f;
      for (int s = 0; s < splits; ++s) v += a.partial[s * stride + (long)m * Ncols + n];
      const float hv = bf16_to_f32(a.resid[(long)m * a.ldr + n]);
      a.out[(long)m * a.ldo + n] = f32_to_bf16(hv + v);
    }
  }
}

template <int BM, int BN>
hipError_t launch_bm_bn(const GemmArgs &a, int epi, int splits, hipStream_t st) {
  const int Ncols = (epi == EPI_SWIGLU) ? 2 * a.N : a.N;
  const int tiles = ((a.M + BM - 1) / BM) * ((Ncols + BN - 1) / BN);
  dim3 grd(tiles, 1, splits), blk(256);
  if (splits > 1) {
    if (epi == EPI_SWIGLU) hipLaunchKernelGGL((k_tiled<BM, BN, EPI_RAW, true>), grd, blk, 0, st, a);
    else hipLaunchKernelGGL((k_tiled<BM, BN, EPI_RAW, false>), grd, blk, 0, st, a);
    return hipGetLastError();
  }
  switch (epi) {
    case EPI_LOGITS: hipLaunchKernelGGL((k_tiled<BM, BN, EPI_LOGITS, false>), grd, blk, 0, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((k_tiled<BM, BN, EPI_SWIGLU, true>), grd, blk, 0, st, a); break;
    case EPI_RESID: hipLaunchKernelGGL((k_tiled<BM, BN, EPI_RESID, false>), grd, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int tiled_slots(int N, int bn) { return ((N + bn - 1) / bn) * 2; }

hipError_t launch_gemm_tiled(const GemmArgs &a, int epi, int bm, int bn, int splits, hipStream_t st) {
  if (bn == 256 && bm == 256) return launch_bm_bn<256, 256>(a, epi, splits, st);
  if (bn != 128) return hipErrorInvalidValue;
  switch (bm) {
    case 64: return launch_bm_bn<64, 128>(a, epi, splits, st);
    case 128: return launch_bm_bn<128, 128>(a, epi, splits, st);
    case 256: return launch_bm_bn<256, 128>(a, epi, splits, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_splitk_reduce(const GemmArgs &a, int epi, int splits, int bn, hipStream_t st) {
  const long total = (long)a.M * a.N;
  long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  dim3 grd((unsigned)blocks), blk(256);
  if (epi == EPI_SWIGLU) hipLaunchKernelGGL((k_splitk_reduce<EPI_SWIGLU>), grd, blk, 0, st, a, splits, bn);
  else if (epi == EPI_RESID) hipLaunchKernelGGL((k_splitk_reduce<EPI_RESID>), grd, blk, 0, st, a, splits, bn);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sv
