/*
 * sv_peaks.h -- achievable-peak probes (libsvpeaks.so), measured beside the vendor peaks
 * of MI355X.  A verification step is priced by the weight bytes it reads at small batch
 * and by its matrix work at large batch ("Let's start over, Misha: speculative decoding
 * from draft to verification", "Why is generation so slow at all?"; "Speculative decoding
 * in production: comparing methods in the Wildberries shopping assistant", "A bit of
 * theory", Statement 3), so the two ceilings that matter are the HBM read rate and the
 * dense bf16 MFMA rate.  Not part of the verification ABI (spec_verify.h).
 *
 * Pointers are device pointers owned by the caller; `stream` is a hipStream_t.  Each call
 * launches one kernel between two events on `stream`, waits for it, and stores the
 * elapsed milliseconds in *ms.  Return 0, or -1 on a bad argument or a HIP error.
 */
#ifndef SV_PEAKS_H
#define SV_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read all `bytes` of `src` once (16-byte nontemporal loads, 1 KiB contiguous per wave
 * load, 16 loads in flight per lane, one 512-thread workgroup per CU).  bytes: a multiple
 * of 16; src 16-byte aligned; out: at least 1024 uint32 (one XOR word per workgroup). */
int sv_probe_read(const void *src, size_t bytes, uint32_t *out, void *stream, float *ms);

/* `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 per wave on register operands,
 * one 4-wave workgroup per CU; *flops receives the FLOPs executed.  out: at least 1024
 * floats (written only to keep the results live; normally untouched). */
int sv_probe_mfma(int iters, float *out, void *stream, float *ms, double *flops);

#ifdef __cplusplus
}
#endif

#endif /* SV_PEAKS_H */
