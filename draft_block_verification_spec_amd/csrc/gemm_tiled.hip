// LDS-tiled MFMA GEMM for larger row counts: out[m, n] = sum_k X[m, k] W[n, k].
//
// Once B*(K+1) rows share each weight read the verification pass stops being
// bound by HBM and becomes compute-bound (Wildberries page, "A bit of theory",
// Statement 3: under load the step time grows with B*(K+1)).  Each 256-thread
// workgroup (2 x 2 waves, or 1 x 4 for 160-row tiles) owns a BM x BN output tile
// and walks k in 64-wide slices.  Both operand slices travel from global memory
// straight into LDS with global_load_lds_dwordx4 (no staging registers), NS slices
// deep, so the loads of future slices run under the MFMAs of the current one.  Inside a row the sixteen-
// byte chunks are XOR-swizzled so the 128-bit operand reads of
// v_mfma_f32_32x32x16_bf16 hit distinct banks.  The LDS reads of the next k step,
// and at slice boundaries the global->LDS loads of a future slice, are interleaved
// one per MFMA.  Workgroups are mapped XCD-major so the row tiles that share a
// weight tile run on one XCD and share its L2.  Split-K writes fp32 partials that a
// second kernel reduces in a fixed order.
#include "sv_device.h"

namespace sv {

namespace {

typedef __attribute__((address_space(3))) void *lds_ptr;

// Slice geometry for a k-slice depth BK: RB bytes per tile row, CPR 16-byte chunks per
// row, RPI rows covered by one wave-wide 1 KB load.
template <int BK>
struct Slice {
  static constexpr int RB = BK * 2, CPR = BK / 8, RPI = 64 / CPR;
  // Row r's logical chunk c sits at chunk c ^ swz(r): with 64 banks of 4 bytes, 16
  // consecutive rows read at one logical chunk then hit 16 distinct 16-byte bank groups.
  static __device__ __forceinline__ int swz(int r) { return (r / (16 / CPR)) & (CPR - 1); }
};

// 16 bytes per lane from global memory into LDS: lane l writes bytes
// [16 l, 16 l + 16) after the wave-uniform LDS address.  Activations stay cached (every
// column tile reads them again); weight slices are read by the few row tiles of one
// column tile at about the same time and never again, so they go nontemporal (cache
// policy operand 2: the NT bit) and leave L2 to the activations (B = 8 LM head
// 269 -> 259 us, wide model step -2%).
__device__ __forceinline__ void dma16(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma16_nt(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr)lds, 16, 0, 2);
}

// Read one accumulator out of its AGPR where it is used, so the compiler does not
// copy every accumulator to VGPRs at once after the main loop.
__device__ __forceinline__ float agpr_read(float x) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
  return v;
}

// s_waitcnt vmcnt(N) alone (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// The four waves of a workgroup as a grid over the tile: 2 x 2 when the rows split into
// two 32-row-aligned halves, otherwise 1 x 4 (all rows, a quarter of the columns each),
// which lets a row tile hold 32 * odd rows (160 rows: 288 rows in two row tiles).
template <int BM, int BN>
struct WaveGrid {
  static constexpr int WN = BM % 64 == 0 ? 2 : 4, WM = 4 / WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of whole 32 x 32 blocks");
};

// Waves per SIMD the kernel is compiled for: one where the slice pipeline's LDS already
// holds the CU to one workgroup (the 192-row shape among them), and for 256 x 256 tiles,
// whose accumulators need the whole register file; two otherwise.
template <int BM, int BN, int BK, int NS>
constexpr int waves_per_eu() {
  return (BM * BN >= 256 * 256 || BM == 192 || (160 * 1024) / (NS * (BM + BN) * BK * 2) < 2) ? 1 : 2;
}

// The epilogue of one BM x BN tile, run by the four MFMA waves (wave (wm, wn) of the
// wave grid owns rows wm*WTM.. and columns wn*WTN..) straight from their accumulators.
template <int BM, int BN, int EPI, bool PAIR>
__device__ __forceinline__ void tile_epilogue(const GemmArgs &a,
                                              f32x16 (&acc)[WaveGrid<BM, BN>::TM][WaveGrid<BM, BN>::TN], int m0,
                                              int n0, int tni, int wm, int wn, int lane, int M, int Ncols, int z) {
  using WG = WaveGrid<BM, BN>;
  constexpr int WTM = WG::WTM, WTN = WG::WTN, TM = WG::TM, TN = WG::TN;
  const int l32 = lane & 31, hi = lane >> 5;
  // ---- epilogue.  Lane l of block (i, j) holds column l%32 and, for register r,
  // row (r/4)*8 + (l/32)*4 + r%4 of the 32x32 block.
  const int rsub = hi * 4;
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
            const float gv = agpr_read(acc[i][2 * jp][r]), uv = agpr_read(acc[i][2 * jp + 1][r]);
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
            a.out[(long)m * a.ldo + n] = f32_to_bf16(hv + agpr_read(acc[i][j][r]));
          }
        }
      }
  } else {  // EPI_LOGITS
    // Logits go out straight from the accumulators.  Row statistics are reduced in
    // registers: each lane folds its TN columns of a row (in increasing column
    // order), then a reduce-scatter over the 32 lanes that share a row group halves
    // the rows per lane at each step, until lanes 2r and 2r+1 hold row r's
    // statistics over all of the wave's columns.
    const bool ws = a.want_s != 0;
    const float invT = a.invT;
    const int pslot = tni * WG::WN + wn;
    const int nb = n0 + wn * WTN + l32;
    if (a.logits) {
      // Nontemporal stores: the logits are read once, by a later kernel, and would
      // otherwise share L2 with the weight tiles (sampled steps 1-3% faster).
      // row bases are wave-uniform; the lane part (row half, column) is an offset
      const long lane_off = (long)rsub * a.ldl + nb;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mrow = m0 + wm * WTM + i * 32 + (r >> 2) * 8 + (r & 3);
          float *rowbase = a.logits + (long)mrow * a.ldl;
          if (mrow + rsub < M) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
              if (nb + j * 32 < a.N) __builtin_nontemporal_store(acc[i][j][r], rowbase + lane_off + j * 32);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      auto fold = [&](int r) {
        float zv[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) zv[j] = (nb + j * 32 < a.N) ? agpr_read(acc[i][j][r]) : -INFINITY;
        float b1 = zv[0];
        int j1 = 0;
#pragma unroll
        for (int j = 1; j < TN; ++j)
          if (zv[j] > b1) {
            b1 = zv[j];
            j1 = j;
          }
        float b2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < TN; ++j) b2 = fmaxf(b2, j == j1 ? -INFINITY : zv[j]);
        float sum = 0.f;
        if (ws && b1 > -INFINITY) {
#pragma unroll
          for (int j = 0; j < TN; ++j) sum += __expf((zv[j] - b1) * invT);
        }
        StatPart q;
        q.b1 = b1;
        q.b2 = b2;
        q.s = sum;
        q.i1 = b1 > -INFINITY ? a.n_off + nb + j1 * 32 : 0x7fffffff;
        return q;
      };
      // first level straight from the folds: lanes with bit 4 set keep rows 8..15
      StatPart p[8];
      {
        const bool up = (lane & 16) != 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const StatPart lo = fold(k), hi8 = fold(8 + k);
          const StatPart keep = up ? hi8 : lo, send = up ? lo : hi8;
          p[k] = stat_merge(keep, stat_shfl_xor(send, 16), invT, ws);
        }
      }
#pragma unroll
      for (int lvl = 1; lvl < 4; ++lvl) {
        const int half = 8 >> lvl, mask = 16 >> lvl;
        const bool up = (lane & mask) != 0;
#pragma unroll
        for (int k = 0; k < half; ++k) {
          const StatPart keep = up ? p[half + k] : p[k];
          const StatPart send = up ? p[k] : p[half + k];
          p[k] = stat_merge(keep, stat_shfl_xor(send, mask), invT, ws);
        }
      }
      const StatPart st = stat_merge(p[0], stat_shfl_xor(p[0], 1), invT, ws);
      const int rr = l32 >> 1;
      const int m = m0 + wm * WTM + i * 32 + (rr >> 2) * 8 + rsub + (rr & 3);
      if ((lane & 1) == 0 && m < M) a.parts[(long)m * a.nslots + pslot] = st;
    }
  }
}

// PAIR: the weight rows of a tile are [32 gate | 32 up] groups of the same outputs.
template <int BM, int BN, int BK, int NS, int EPI, bool PAIR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(waves_per_eu<BM, BN, BK, NS>(), waves_per_eu<BM, BN, BK, NS>())))
void k_tiled(const GemmArgs a) {
  constexpr int RB = Slice<BK>::RB, CPR = Slice<BK>::CPR, RPI = Slice<BK>::RPI;
  constexpr int SA = BM * RB, SB = BN * RB, SS = SA + SB;  // bytes of one slice
  constexpr int IA = BM / RPI / 4, IB = BN / RPI / 4;      // 1 KB loads per wave per slice
  using WG = WaveGrid<BM, BN>;
  constexpr int WTM = WG::WTM, WTN = WG::WTN, TM = WG::TM, TN = WG::TN;
  constexpr int KS = BK / 16;
  static_assert(IA >= 1 && IB >= 1, "tile too small");
  static_assert(NS >= 2 && (NS - 1) * (IA + IB) < 64, "slice pipeline depth");
  static_assert(KS % 2 == 0, "fragment sets alternate within a slice");
  static_assert(!PAIR || (WTN % 64) == 0, "paired tiles need gate/up block pairs");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * SS];

  if (a.status_reset && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) *a.status_reset = 0;
  if (a.counter_reset && blockIdx.x == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < max(1, a.counter_reset_n); i += blockDim.x) a.counter_reset[i] = 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WG::WN, wn = wave % WG::WN;
  const int M = live_rows(a);
  if (M < 0) return;  // another launch of the same product does the work
  if (a.nslots_out && blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) *a.nslots_out = a.nslots_plan;
  const int Ncols = PAIR ? 2 * a.N : a.N;  // columns of the weight-row space
  // Only row tiles that hold rows are walked: with a device-side row count below a.M the
  // live tiles still spread over every workgroup (skipping the dead ones in place would
  // leave all live tiles to the workgroups whose slot meets them, half the grid at two
  // row tiles).
  const int tiles_m = M > 0 ? (M + BM - 1) / BM : 0;
  const int total = tiles_m * ((Ncols + BN - 1) / BN);
  const int splits = gridDim.z, z = blockIdx.z;
  const int nkt_total = a.K / BK;
  const int per = (nkt_total + splits - 1) / splits;
  const int kt0 = z * per;
  const int kt1 = min(nkt_total, kt0 + per);
  const int nkt = kt1 > kt0 ? kt1 - kt0 : 0;
  // Tiles: workgroup w takes tiles r*G + slot(w), r = 0, 1, ... (one round when the grid
  // covers every tile).  With G a multiple of 8, workgroup w runs on XCD w % 8 and
  // slot(w) = (w % 8) * G/8 + w / 8, so consecutive tiles - the row tiles of one weight
  // tile - run on one XCD at the same time and read that weight tile through its L2.
  // A persistent grid (one workgroup per CU slot) keeps those row tiles in step round
  // after round; the hardware dispatcher would start them at scattered times.
  const int G = gridDim.x;
  const int slot = (G & 7) == 0 ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  for (int lin = slot; lin < total; lin += G) {
  const int tmi = lin % tiles_m, tni = lin / tiles_m;
  const int m0 = tmi * BM, n0 = tni * BN;
  if (m0 >= M) continue;
  if (lin != slot) {  // every wave's reads of the previous tile's slices are done
    lgkm_wait0();
    __builtin_amdgcn_s_barrier();
  }

  // Per-lane global sources of the slice loads.  Load j of this wave fills LDS bytes
  // [(wave + 4 j) KB, +1 KB) of the operand: rows (wave + 4 j) * RPI + lane / CPR, at
  // swizzled chunk lane % CPR.  Rows past M (or N) read a clamped valid row; their
  // results are never stored.
  const uint16_t *ga[IA];
  const uint16_t *gb[IB];
  const int mlast = max(M, 1) - 1;
#pragma unroll
  for (int j = 0; j < IA; ++j) {
    const int r = (wave + 4 * j) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ Slice<BK>::swz(r);
    const int m = min(m0 + r, mlast);
    ga[j] = (m < a.m1 ? a.x1 + (long)m * a.ldx1 : a.x2 + (long)(m - a.m1) * a.ldx2) + c * 8;
  }
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const int r = (wave + 4 * j) * RPI + lane / CPR;
    const int c = (lane % CPR) ^ Slice<BK>::swz(r);
    if constexpr (PAIR) {
      const int p = r >> 6, half = (r >> 5) & 1, rr = r & 31;
      const int n = min((n0 >> 1) + p * 32 + rr, a.N - 1);
      gb[j] = (half ? a.w2 : a.w) + (long)n * a.K + c * 8;
    } else {
      const int n = min(n0 + r, a.N - 1);
      gb[j] = a.w + (long)n * a.K + c * 8;
    }
  }
  // element offset of slice t of this split; past the end it re-reads the last slice
  auto kofs = [&](int t) -> long { return (long)(kt0 + min(t, nkt - 1)) * BK; };
  auto issue_one = [&](long ko, uint32_t soff, int g) {
    uint8_t *sb = smem + soff;
    if (g < IA) dma16(ga[g] + ko, sb + (wave + 4 * g) * 1024);
    else dma16_nt(gb[g - IA] + ko, sb + SA + (wave + 4 * (g - IA)) * 1024);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int l32 = lane & 31, hi = lane >> 5;
  // lane l reads row l%32 of a 32-row block at logical chunk 2 kk + l/32 of k step kk
  int off[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) off[kk] = l32 * RB + (((kk * 2 + hi) ^ Slice<BK>::swz(l32)) << 4);
  bf16x8 af[2][TM], bfr[2][TN];
  auto lfrag_one = [&](int set, uint32_t soff, int kk, int g) {
    const uint8_t *sb = smem + soff;
    if (g < TM) af[set][g] = *reinterpret_cast<const bf16x8 *>(sb + (wm * WTM + g * 32) * RB + off[kk]);
    else bfr[set][g - TM] = *reinterpret_cast<const bf16x8 *>(sb + SA + (wn * WTN + (g - TM) * 32) * RB + off[kk]);
  };
  // One k step: TM*TN MFMAs on fragment set `cur`; after MFMA q comes the LDS read of
  // fragment q of the next step and, at a slice boundary, global->LDS load q.
  auto step = [&](int cur, uint32_t rsoff, int rkk, bool ld, long ko, uint32_t lsoff) {
#pragma unroll
    for (int q = 0; q < TM * TN; ++q) {
      const int i = q / TN, j = q % TN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
      if (ld && q < IA + IB) issue_one(ko, lsoff, q);
      if (q < TM + TN) lfrag_one(cur ^ 1, rsoff, rkk, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ld) {  // loads left over when a slice needs more loads than the step has MFMAs
#pragma unroll
      for (int g = TM * TN; g < IA + IB; ++g) issue_one(ko, lsoff, g);
    }
#pragma unroll
    for (int g = TM * TN; g < TM + TN; ++g) lfrag_one(cur ^ 1, rsoff, rkk, g);
  };

  if (nkt > 0) {
    // prologue: slices 0 .. NS-1 in flight, wait for slice 0
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int g = 0; g < IA + IB; ++g) issue_one(kofs(s), s * SS, g);
    }
    vm_wait<(NS - 1) * (IA + IB)>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int g = 0; g < TM + TN; ++g) lfrag_one(0, 0, 0, g);

    uint32_t scur = 0;
    for (int t = 0; t < nkt; ++t) {
      const uint32_t snext = scur + SS == NS * SS ? 0 : scur + SS;
#pragma unroll
      for (int kk = 0; kk + 1 < KS; ++kk) step(kk & 1, scur, kk + 1, false, 0, 0);
      // Slice boundary: every wave has finished reading slice t (its LDS reads are
      // complete), slice t+1 has landed.  Refill slice t's buffer with slice t+NS and
      // start reading slice t+1.  After the last slice this reads a stale buffer that
      // no MFMA consumes.
      lgkm_wait0();
      vm_wait<(NS - 2) * (IA + IB)>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      step((KS - 1) & 1, snext, 0, true, kofs(t + NS), scur);
      scur = snext;
    }
    // no load may still be writing LDS when the workgroup leaves
    vm_wait<0>();
  }

  tile_epilogue<BM, BN, EPI, PAIR>(a, acc, m0, n0, tni, wm, wn, lane, M, Ncols, z);
  }  // tiles
}

// Fixed-order reduction of split-K partials followed by the elementwise epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void k_splitk_reduce(const GemmArgs a, int splits, int bn) {
  const int M = live_rows(a);
  if (M < 0) return;
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

// Workgroups of one tile shape resident per CU: bounded by the LDS of the slice pipeline
// (160 KiB per CU) and by the waves per SIMD the kernel is compiled for.
template <int BM, int BN, int BK, int NS>
constexpr int per_cu() {
  constexpr int lds = NS * (BM + BN) * BK * 2;
  constexpr int by_lds = (160 * 1024) / lds;
  return by_lds < waves_per_eu<BM, BN, BK, NS>() ? by_lds : waves_per_eu<BM, BN, BK, NS>();
}

template <int BM, int BN, int BK, int NS>
hipError_t launch_shape(const GemmArgs &a, int epi, int splits, hipStream_t st) {
  const int Ncols = (epi == EPI_SWIGLU) ? 2 * a.N : a.N;
  const int tiles = ((a.M + BM - 1) / BM) * ((Ncols + BN - 1) / BN);
  // more tiles than resident slots: a persistent grid of one workgroup per slot
  int gx = tiles;
  const int slots = (per_cu<BM, BN, BK, NS>() * num_cus()) & ~7;
  if (splits == 1 && slots > 0 && tiles > slots) gx = slots;
  dim3 grd(gx, 1, splits), blk(256);
  // paired gate/up tiles need whole 64-row (gate | up) groups per wave column
  constexpr bool pair_ok = WaveGrid<BM, BN>::WTN % 64 == 0;
  if (splits > 1) {
    if constexpr (pair_ok) {
      if (epi == EPI_SWIGLU) {
        hipLaunchKernelGGL((k_tiled<BM, BN, BK, NS, EPI_RAW, true>), grd, blk, 0, st, a);
        return hipGetLastError();
      }
    } else {
      if (epi == EPI_SWIGLU) return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((k_tiled<BM, BN, BK, NS, EPI_RAW, false>), grd, blk, 0, st, a);
    return hipGetLastError();
  }
  switch (epi) {
    case EPI_LOGITS: hipLaunchKernelGGL((k_tiled<BM, BN, BK, NS, EPI_LOGITS, false>), grd, blk, 0, st, a); break;
    case EPI_SWIGLU:
      if constexpr (pair_ok) hipLaunchKernelGGL((k_tiled<BM, BN, BK, NS, EPI_SWIGLU, true>), grd, blk, 0, st, a);
      else return hipErrorInvalidValue;
      break;
    case EPI_RESID: hipLaunchKernelGGL((k_tiled<BM, BN, BK, NS, EPI_RESID, false>), grd, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int tiled_slots(int N, const TileShape &sh) { return ((N + sh.bn - 1) / sh.bn) * (sh.bm % 64 == 0 ? 2 : 4); }

// Shapes measured best on MI355X for the row counts of the verification step (LM head,
// gate/up, down at d = 4096 and 8192): the fewer the rows, the more of each slice is
// weights, and the deeper the pipeline must be to keep HBM busy.
TileShape tiled_shape(int M, int N, int K, int epi) {
  const bool k128 = K % 128 == 0;
  if (epi == EPI_SWIGLU) {
    if (M <= 128) return TileShape{128, 128, 64, 4};
    // 129-160 rows: 160 x 256 tiles move 52 KiB per slice against 40 KiB for 192 x 128
    // ones but cover twice the columns; taken when that needs fewer slice-rounds over the
    // CUs (d_ff = 28672: one round against two, step 0.80 -> 0.77 ms; d_ff = 12288: one
    // round either way, 192 x 128 keeps 192 CUs busy instead of 96)
    if (M <= 160) {
      const long cus = num_cus();
      const long r160 = ((2L * N + 255) / 256 + cus - 1) / cus, r192 = ((2L * N + 127) / 128 + cus - 1) / cus;
      if (13 * r160 < 10 * r192) return TileShape{160, 256, 64, 3};
    }
    // one row tile, at most a third empty (160 rows at d = 8192: 219 us against 239 us
    // for 256 x 256 tiles)
    if (M <= 192) return TileShape{192, 128, 64, 3};
    // two 128-row tiles at 193-256 rows (256 rows: 0.7% of the step faster than 256 x 128)
    if (M <= 256) return TileShape{128, 256, 64, 3};
    // 256-row tiles, one workgroup per CU either way: 256 x 256 when it needs enough fewer
    // rounds over the CUs than 256 x 128 (a 256 x 256 tile takes ~1.7x as long as a
    // 256 x 128 one), e.g. 512 rows: 192 tiles in one round against 384 tiles in two
    const long tm = (M + 255) / 256, cus = num_cus();
    const long r128 = (tm * ((2L * N + 127) / 128) + cus - 1) / cus;
    const long r256 = (tm * ((2L * N + 255) / 256) + cus - 1) / cus;
    return 10 * r128 <= 17 * r256 ? TileShape{256, 128, 64, 3} : TileShape{256, 256, 64, 2};
  }
  if (epi == EPI_RESID) {
    if (M <= 64) return k128 ? TileShape{64, 128, 128, 3} : TileShape{64, 128, 64, 2};
    // 129-160 rows: 160 x 256 tiles when their split-K workgroups still fill the CUs
    // (the wide model's 8192 outputs: 32 tiles x 8 splits), else one 192-row tile.  The
    // split bound is the one the planner applies: at most 8, and at least 4 slices each.
    if (M > 128 && M <= 160) {
      const int maxs = K / 64 / 4 < 8 ? K / 64 / 4 : 8;
      if ((long)((N + 255) / 256) * maxs >= num_cus()) return TileShape{160, 256, 64, 3};
    }
    if (M > 128 && M <= 192) return TileShape{192, 128, 64, 3};  // 160 rows: 121 us against 149 us
    return M <= 256 ? TileShape{128, 256, 64, 3} : TileShape{256, 128, 64, 3};
  }
  // (a single 320 x 128 row tile at 288 rows measured 9% slower than three 128 x 256 ones;
  // at 256 rows two 128 x 256 row tiles beat one 256 x 128 row tile by 4% of the step)
  // 129-160 and 257-320 rows: one or two row tiles of 160 x 256 (160 rows: LM head
  // 0.55 -> 0.44 ms for the d = 8192 model, 364 -> 358 us at d = 4096; 288 rows: 0.86 ->
  // 0.76 ms against three 128 x 256 row tiles); 161-192 rows: one 192 x 192 row tile
  // (192 rows: 367 -> 358 us against 256 x 128 tiles).  193-256 rows: one 256 x 256 row
  // tile, which moves 2 bytes into LDS per weight byte against 3 for two 128 x 256 row
  // tiles (the rate into LDS is what these kernels are held to); with the ragged columns
  // on 256 x 128 tiles (the planner's split) the V = 151936 head at 256 rows went from
  // 378 to 351 us, at 224 rows from 376 to 349 us.
  if (M <= 64) return k128 ? TileShape{64, 128, 128, 3} : TileShape{64, 128, 64, 2};
  if (M <= 128) return TileShape{128, 128, 64, 4};
  if (M <= 160) return TileShape{160, 256, 64, 3};
  if (M <= 192) return TileShape{192, 192, 64, 3};
  if (M <= 256) return TileShape{256, 256, 64, 2};
  if (M <= 320) return TileShape{160, 256, 64, 3};
  if (M <= 384) return TileShape{128, 256, 64, 3};
  return TileShape{256, 256, 64, 2};
}

#define SV_TILE_SHAPES(X) \
  X(64, 128, 64, 2)       \
  X(64, 128, 128, 3)      \
  X(128, 128, 64, 4)      \
  X(192, 128, 64, 3)      \
  X(256, 128, 64, 3)      \
  X(128, 256, 64, 3)      \
  X(160, 256, 64, 3)      \
  X(192, 192, 64, 3)      \
  X(256, 256, 64, 2)

int tiled_per_cu(const TileShape &sh) {
#define SV_PER_CU(BM, BN, BK, NS) \
  if (sh.bm == BM && sh.bn == BN && sh.bk == BK && sh.ns == NS) return per_cu<BM, BN, BK, NS>();
  SV_TILE_SHAPES(SV_PER_CU)
#undef SV_PER_CU
  return 0;
}

hipError_t launch_gemm_tiled(const GemmArgs &a, int epi, const TileShape &sh, int splits, hipStream_t st) {
  if (a.K % sh.bk != 0 || a.K < sh.bk) return hipErrorInvalidValue;
#define SV_LAUNCH(BM, BN, BK, NS) \
  if (sh.bm == BM && sh.bn == BN && sh.bk == BK && sh.ns == NS) return launch_shape<BM, BN, BK, NS>(a, epi, splits, st);
  SV_TILE_SHAPES(SV_LAUNCH)
#undef SV_LAUNCH
  return hipErrorInvalidValue;
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
