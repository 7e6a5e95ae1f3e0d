// Device-side helpers shared by the kernels of libspecverify (gfx950, wave64).
#pragma once

#include "sv_internal.h"

namespace sv {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Rows of a launch: a.M, or the device-side count when one is given.  A launch gated
// to a range of device-side counts (m_lo < count <= m_hi) gets -1 outside it.
__device__ __forceinline__ int live_rows(const GemmArgs &a) {
  if (!a.M_dev) return a.M;
  const int md = *a.M_dev;
  if (md <= a.m_lo || (a.m_hi > 0 && md > a.m_hi)) return -1;
  return min(a.M, md);
}


__device__ __forceinline__ u32x4 ld_nt(const uint16_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ StatPart stat_empty() {
  StatPart s;
  s.b1 = -INFINITY;
  s.b2 = -INFINITY;
  s.s = 0.f;
  s.i1 = 0x7fffffff;
  return s;
}

// Fold one value z at column n into running statistics.  Columns must arrive in
// increasing order per accumulator for the lowest-index tie rule to hold; merges
// use the explicit index comparison.
__device__ __forceinline__ void stat_push(StatPart &st, float z, int n, float invT, bool want_s) {
  if (z > st.b1) {
    if (want_s) st.s = st.s * __expf((st.b1 - z) * invT) + 1.f;
    st.b2 = st.b1;
    st.b1 = z;
    st.i1 = n;
  } else {
    if (want_s) st.s += __expf((z - st.b1) * invT);
    st.b2 = fmaxf(st.b2, z);
  }
}

__device__ __forceinline__ StatPart stat_merge(const StatPart &a, const StatPart &b, float invT,
                                               bool want_s) {
  StatPart r;
  r.b1 = fmaxf(a.b1, b.b1);
  r.i1 = (a.b1 > b.b1) ? a.i1 : (b.b1 > a.b1) ? b.i1 : min(a.i1, b.i1);
  r.b2 = fmaxf(fminf(a.b1, b.b1), fmaxf(a.b2, b.b2));
  if (want_s) {
    float sa = (a.s > 0.f) ? a.s * __expf((a.b1 - r.b1) * invT) : 0.f;
    float sb = (b.s > 0.f) ? b.s * __expf((b.b1 - r.b1) * invT) : 0.f;
    r.s = sa + sb;
  } else {
    r.s = 0.f;
  }
  return r;
}

// Butterfly merge over `width` consecutive lanes (width a power of two <= 64).
__device__ __forceinline__ StatPart stat_shfl_xor(const StatPart &s, int mask) {
  StatPart o;
  o.b1 = __shfl_xor(s.b1, mask);
  o.b2 = __shfl_xor(s.b2, mask);
  o.s = __shfl_xor(s.s, mask);
  o.i1 = __shfl_xor(s.i1, mask);
  return o;
}

}  // namespace sv
