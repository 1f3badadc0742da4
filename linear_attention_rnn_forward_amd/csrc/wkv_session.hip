// Session state save and resume ([multigrid] = multigrid.ai rwkv, "The state,
// in bytes", and the closing note on serialising a session): the recurrent
// state of one sequence -- a, b, p of every layer plus the shifted token(s)
// of the previous step -- copied between a decode batch [L,S,C] on the device
// and a host blob, so that a session can be stored and resumed elsewhere.
//
// Blob layout (little-endian, as the host writes it):
//   header  (64 bytes): magic "WKVS", format version, L, C, dtype, n_shift
//   a, b, p  [L][C] fp32 each
//   shift    n_shift arrays [L][C] in the I/O dtype
// Host code only: the copies are hipMemcpy2DAsync on the caller's stream.
#include "wkv.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <string>

namespace {

constexpr uint32_t kMagic = 0x53564B57u;  // "WKVS"
constexpr uint32_t kVersion = 1;
constexpr size_t kHeaderBytes = 64;

struct Header {
    uint32_t magic;
    uint32_t version;
    int64_t L;
    int64_t C;
    int32_t dtype;
    int32_t n_shift;
    uint8_t reserved[kHeaderBytes - 32];
};
static_assert(sizeof(Header) == kHeaderBytes, "header is 64 bytes");

size_t esize(int dtype) { return dtype == WKV_BF16 ? 2 : 4; }

bool sizes_ok(int64_t L, int64_t C, int dtype, int n_shift) {
    if (L < 1 || C < 1 || n_shift < 0 || n_shift > WKV_SESSION_MAX_SHIFT) return false;
    if (dtype != WKV_F32 && dtype != WKV_BF16) return false;
    if (L > (int64_t(1) << 40) / C) return false;  // keeps the byte counts in range
    return true;
}

size_t blob_bytes(int64_t L, int64_t C, int dtype, int n_shift) {
    return kHeaderBytes + size_t(L) * size_t(C) * (12 + size_t(n_shift) * esize(dtype));
}

}  // namespace

// Error reporting is shared with wkv_api.hip through these two calls.
namespace wkv_detail {
int fail_status(int status, const char* msg);
int ok_status();
}  // namespace wkv_detail

extern "C" {

size_t wkv_session_bytes(int64_t L, int64_t C, int dtype, int n_shift) {
    if (!sizes_ok(L, C, dtype, n_shift)) return 0;
    return blob_bytes(L, C, dtype, n_shift);
}

int wkv_session_save(int64_t L, int64_t S, int64_t C, int dtype, int64_t seq, const float* a,
                     const float* b, const float* p, const void* const* shift, int n_shift,
                     void* blob, size_t blob_size, void* stream) {
    using wkv_detail::fail_status;
    if (!sizes_ok(L, C, dtype, n_shift) || S < 1)
        return fail_status(WKV_ERR_SHAPE, "invalid L, S, C, dtype or n_shift");
    if (seq < 0 || seq >= S) return fail_status(WKV_ERR_ARG, "seq out of range [0, S)");
    if (!a || !b || !p || !blob || (n_shift > 0 && !shift))
        return fail_status(WKV_ERR_NULL, "a, b, p, blob (and shift when n_shift > 0) are required");
    for (int i = 0; i < n_shift; i++)
        if (!shift[i]) return fail_status(WKV_ERR_NULL, "a shift array is NULL");
    const size_t need = blob_bytes(L, C, dtype, n_shift);
    if (blob_size < need) return fail_status(WKV_ERR_ARG, "blob too small for this state");

    Header h;
    std::memset(&h, 0, sizeof h);
    h.magic = kMagic;
    h.version = kVersion;
    h.L = L;
    h.C = C;
    h.dtype = dtype;
    h.n_shift = n_shift;
    char* out = static_cast<char*>(blob);
    std::memcpy(out, &h, sizeof h);
    hipStream_t s = static_cast<hipStream_t>(stream);
    size_t off = kHeaderBytes;
    const float* st[3] = {a, b, p};
    for (const float* src : st) {
        hipError_t e = hipMemcpy2DAsync(out + off, size_t(C) * 4, src + seq * C, size_t(S * C) * 4,
                                        size_t(C) * 4, size_t(L), hipMemcpyDeviceToHost, s);
        if (e != hipSuccess) return fail_status(WKV_ERR_HIP, hipGetErrorString(e));
        off += size_t(L) * size_t(C) * 4;
    }
    const size_t es = esize(dtype);
    for (int i = 0; i < n_shift; i++) {
        const char* src = static_cast<const char*>(shift[i]) + size_t(seq * C) * es;
        hipError_t e = hipMemcpy2DAsync(out + off, size_t(C) * es, src, size_t(S * C) * es,
                                        size_t(C) * es, size_t(L), hipMemcpyDeviceToHost, s);
        if (e != hipSuccess) return fail_status(WKV_ERR_HIP, hipGetErrorString(e));
        off += size_t(L) * size_t(C) * es;
    }
    return wkv_detail::ok_status();
}

int wkv_session_load(int64_t L, int64_t S, int64_t C, int dtype, int64_t seq, const void* blob,
                     size_t blob_size, float* a, float* b, float* p, void* const* shift, int n_shift,
                     void* stream) {
    using wkv_detail::fail_status;
    if (!sizes_ok(L, C, dtype, n_shift) || S < 1)
        return fail_status(WKV_ERR_SHAPE, "invalid L, S, C, dtype or n_shift");
    if (seq < 0 || seq >= S) return fail_status(WKV_ERR_ARG, "seq out of range [0, S)");
    if (!a || !b || !p || !blob || (n_shift > 0 && !shift))
        return fail_status(WKV_ERR_NULL, "a, b, p, blob (and shift when n_shift > 0) are required");
    for (int i = 0; i < n_shift; i++)
        if (!shift[i]) return fail_status(WKV_ERR_NULL, "a shift array is NULL");
    if (blob_size < kHeaderBytes) return fail_status(WKV_ERR_ARG, "blob shorter than its header");
    Header h;
    std::memcpy(&h, blob, sizeof h);
    if (h.magic != kMagic) return fail_status(WKV_ERR_ARG, "not a session blob (bad magic)");
    if (h.version != kVersion) return fail_status(WKV_ERR_UNSUPPORTED, "unknown session blob version");
    if (h.L != L || h.C != C || h.dtype != dtype || h.n_shift != n_shift)
        return fail_status(WKV_ERR_ARG, "session blob was saved with another L, C, dtype or n_shift");
    const size_t need = blob_bytes(L, C, dtype, n_shift);
    if (blob_size < need) return fail_status(WKV_ERR_ARG, "blob shorter than its contents");

    const char* in = static_cast<const char*>(blob);
    hipStream_t s = static_cast<hipStream_t>(stream);
    size_t off = kHeaderBytes;
    float* st[3] = {a, b, p};
    for (float* dst : st) {
        hipError_t e = hipMemcpy2DAsync(dst + seq * C, size_t(S * C) * 4, in + off, size_t(C) * 4,
                                        size_t(C) * 4, size_t(L), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return fail_status(WKV_ERR_HIP, hipGetErrorString(e));
        off += size_t(L) * size_t(C) * 4;
    }
    const size_t es = esize(dtype);
    for (int i = 0; i < n_shift; i++) {
        char* dst = static_cast<char*>(shift[i]) + size_t(seq * C) * es;
        hipError_t e = hipMemcpy2DAsync(dst, size_t(S * C) * es, in + off, size_t(C) * es,
                                        size_t(C) * es, size_t(L), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return fail_status(WKV_ERR_HIP, hipGetErrorString(e));
        off += size_t(L) * size_t(C) * es;
    }
    return wkv_detail::ok_status();
}

}  // extern "C"
