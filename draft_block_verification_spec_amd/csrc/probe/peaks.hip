// Achievable-peak probes for MI355X (gfx950), reported beside the vendor peaks.
//
// A verification step is priced by the weight bytes it reads at small batch and by its
// matrix work at large batch ("Let's start over, Misha", "Why is generation so slow at
// all?"; Wildberries page, "A bit of theory", Statement 3).  These two kernels measure what
// the part actually delivers for each:
//  * sv_probe_read: every byte of a device buffer read once with 16-byte nontemporal
//    loads, each wave streaming 4 rows x 256 contiguous bytes per load and keeping 16
//    loads in flight (the access shape of the weight-streaming GEMM);
//  * sv_probe_mfma: back-to-back independent v_mfma_f32_32x32x16_bf16 on register
//    operands, no memory traffic, one wave per SIMD.
// Both return the elapsed time of the launch measured with events on `stream`; the host
// computes bytes/s or FLOP/s.  Not part of the verification library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_peaks.h"

#define SV_PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int READ_THREADS = 512;
constexpr int READ_INFLIGHT = 16;  // 16-byte loads in flight per lane

// Workgroup g reads chunks g, g + G, ... of 512 threads x 16 loads x 16 bytes (128 KiB); a
// lane's load i covers bytes [((i * 512 + tid) * 16), +16) of the chunk, so each wave load
// is 1 KiB contiguous.  The XOR of everything read goes to out[g] so no load is dropped.
__global__ __launch_bounds__(READ_THREADS) void k_probe_read(const u32x4 *src, size_t n16, uint32_t *out) {
  const size_t chunk = (size_t)READ_THREADS * READ_INFLIGHT;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t base = (size_t)blockIdx.x * chunk; base < n16; base += (size_t)gridDim.x * chunk) {
    u32x4 v[READ_INFLIGHT];
#pragma unroll
    for (int i = 0; i < READ_INFLIGHT; ++i) {
      const size_t idx = base + (size_t)i * READ_THREADS + threadIdx.x;
      v[i] = idx < n16 ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < READ_INFLIGHT; ++i) acc ^= v[i];
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  __shared__ uint32_t red[READ_THREADS / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < READ_THREADS / 64; ++w) t ^= red[w];
    out[blockIdx.x] = t;
  }
}

// Each wave keeps 8 independent 32x32 accumulators and issues `iters` rounds of 8 MFMAs.
// The operands are derived from the thread index so the compiler cannot fold them.
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float *out) {
  const int t = threadIdx.x;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((t + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((t * 3 + i) & 7));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (s == 12345.678f) out[blockIdx.x] = s;  // keeps the accumulators live; never true for these operands
}

int g_cus() {
  int dev = 0;
  hipDeviceProp_t p;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess) return 256;
  return p.multiProcessorCount > 0 ? p.multiProcessorCount : 256;
}

int timed(void (*launch)(void *), void *arg, hipStream_t st, float *ms) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -1;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return -1;
  }
  int rc = 0;
  if (hipEventRecord(e0, st) != hipSuccess) rc = -1;
  if (!rc) launch(arg);
  if (!rc && hipGetLastError() != hipSuccess) rc = -1;
  if (!rc && hipEventRecord(e1, st) != hipSuccess) rc = -1;
  if (!rc && hipEventSynchronize(e1) != hipSuccess) rc = -1;
  if (!rc && hipEventElapsedTime(ms, e0, e1) != hipSuccess) rc = -1;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return rc;
}

struct ReadArgs {
  const void *src;
  size_t bytes;
  uint32_t *out;
  int grid;
  hipStream_t st;
};
void launch_read(void *p) {
  ReadArgs *a = static_cast<ReadArgs *>(p);
  hipLaunchKernelGGL(k_probe_read, dim3(a->grid), dim3(READ_THREADS), 0, a->st,
                     static_cast<const u32x4 *>(a->src), a->bytes / 16, a->out);
}

struct MfmaArgs {
  int iters;
  float *out;
  int grid;
  hipStream_t st;
};
void launch_mfma(void *p) {
  MfmaArgs *a = static_cast<MfmaArgs *>(p);
  hipLaunchKernelGGL(k_probe_mfma, dim3(a->grid), dim3(256), 0, a->st, a->iters, a->out);
}

}  // namespace

SV_PROBE_API int sv_probe_read(const void *src, size_t bytes, uint32_t *out, void *stream, float *ms) {
  if (!src || !out || !ms || bytes < 16 || bytes % 16 || ((uintptr_t)src & 15)) return -1;
  ReadArgs a{src, bytes, out, g_cus(), static_cast<hipStream_t>(stream)};
  return timed(launch_read, &a, a.st, ms);
}

SV_PROBE_API int sv_probe_mfma(int iters, float *out, void *stream, float *ms, double *flops) {
  if (iters < 1 || !out || !ms || !flops) return -1;
  const int grid = g_cus();  // one 4-wave workgroup per CU: one wave per SIMD
  MfmaArgs a{iters, out, grid, static_cast<hipStream_t>(stream)};
  *flops = 2.0 * 32 * 32 * 16 * 8.0 * iters * 4.0 * grid;
  return timed(launch_mfma, &a, a.st, ms);
}
