/*
 * wkv_synth.h -- C ABI of libwkv_synth: device-side generation of seeded
 * synthetic inputs for workloads too large to generate on the host.
 *
 * Input generation only; it is not part of the WKV library.  The generator is
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
 * as 1, 2, 3", SC 2011) with key (seed, key_hi) and counter
 * (ctr_lo, ctr_hi, stream_id, 0); its four output words give eight 16-bit
 * integers whose sum S becomes fl32(S - 262140) * scale (standardised
 * Irwin-Hall(8) when scale = fl32(sqrt(1.5) / 65536)).
 *
 * synth_fill_normal writes the dense array out[n0][n1][n2][n3] (device
 * pointer, fp32), where element (i0,i1,i2,i3) uses the 64-bit counter
 *   base + i0*s0 + i1*s1 + i2*s2 + i3*s3.
 * Enqueued on `stream` (a hipStream_t); returns 0, or a negative value for
 * bad arguments (-1, -2) or a launch failure (-3).
 */
#ifndef WKV_SYNTH_H
#define WKV_SYNTH_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif
int synth_fill_normal(float *out, int64_t n0, int64_t n1, int64_t n2, int64_t n3,
                      int64_t s0, int64_t s1, int64_t s2, int64_t s3, uint64_t base,
                      uint32_t stream_id, uint32_t seed, uint32_t key_hi, float scale,
                      void *stream);
#ifdef __cplusplus
}
#endif
#endif
