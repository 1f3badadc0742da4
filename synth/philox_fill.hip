// Device generator for large synthetic inputs: Philox4x32-10 (Salmon, Moraes,
// Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) and the
// standardised Irwin-Hall(8) transform described in synth/__init__.py.  The
// host side implements the same definitions; tests compare the two bit for
// bit.  This is input generation only: it computes nothing of the WKV method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv_synth.h"

namespace {

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; r++) {
        if (r) {
            k0 += W0;
            k1 += W1;
        }
        const uint32_t hi0 = __umulhi(M0, c[0]), lo0 = M0 * c[0];
        const uint32_t hi1 = __umulhi(M1, c[2]), lo1 = M1 * c[2];
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

__global__ void fill_normal_kernel(float* out, int64_t n1, int64_t n2, int64_t n3, int64_t total,
                                   int64_t s0, int64_t s1, int64_t s2, int64_t s3, uint64_t base,
                                   uint32_t stream, uint32_t seed, uint32_t key_hi, float scale) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t i3 = i % n3;
    const int64_t i2 = (i / n3) % n2;
    const int64_t i1 = (i / (n3 * n2)) % n1;
    const int64_t i0 = i / (n3 * n2 * n1);
    const uint64_t ctr = base + uint64_t(i0 * s0 + i1 * s1 + i2 * s2 + i3 * s3);
    uint32_t c[4] = {uint32_t(ctr), uint32_t(ctr >> 32), stream, 0u};
    philox4x32_10(c, seed, key_hi);
    int32_t s = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) s += int32_t(c[q] & 0xffffu) + int32_t(c[q] >> 16);
    out[i] = float(s - 262140) * scale;
}

}  // namespace

extern "C" int synth_fill_normal(float* out, int64_t n0, int64_t n1, int64_t n2, int64_t n3,
                                 int64_t s0, int64_t s1, int64_t s2, int64_t s3, uint64_t base,
                                 uint32_t stream_id, uint32_t seed, uint32_t key_hi, float scale,
                                 void* stream) {
    if (!out || n0 < 0 || n1 < 1 || n2 < 1 || n3 < 1) return -1;
    const int64_t total = n0 * n1 * n2 * n3;
    if (total == 0) return 0;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 2147483647LL) return -2;
    hipLaunchKernelGGL(fill_normal_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), out, n1, n2, n3, total, s0, s1, s2, s3,
                       base, stream_id, seed, key_hi, scale);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
