// C ABI of libwkv (declared in include/wkv.h): argument validation, path
// selection and launch.  No call allocates memory or synchronises.
#include "wkv.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "wkv_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return WKV_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(WKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// a*b*c without int64 overflow (all >= 0)
bool mul3(int64_t a, int64_t b, int64_t c, int64_t* out) {
    __int128 r = (__int128)a * b;
    if (r > INT64_MAX) return false;
    r *= c;
    if (r > INT64_MAX) return false;
    *out = (int64_t)r;
    return true;
}

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

Range rng(const char* name, const void* p, int64_t bytes) {
    Range r;
    r.name = name;
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + (p ? uintptr_t(bytes) : 0);
    return r;
}

bool overlap(const Range& a, const Range& b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t esize(int dtype) { return dtype == WKV_BF16 ? 2 : 4; }

// outputs may coincide exactly with the input of the same role (in place) but
// must not overlap any other array
int check_state_aliasing(const Range* outs, int nouts, const Range* ins, int nins, bool same_role_ok) {
    for (int i = 0; i < nouts; i++) {
        for (int j = 0; j < nins; j++) {
            if (!overlap(outs[i], ins[j])) continue;
            const bool exact = outs[i].lo == ins[j].lo && outs[i].hi == ins[j].hi;
            if (same_role_ok && exact && i == j) continue;
            return fail(WKV_ERR_ALIAS, "%s overlaps %s", outs[i].name, ins[j].name);
        }
        for (int j = 0; j < i; j++)
            if (overlap(outs[i], outs[j]))
                return fail(WKV_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    return WKV_OK;
}

// Bytes of the saved states of a [B, T, C] problem: fp32 [B][ceil(T/16)][2][C].
int64_t saved_state_bytes(int64_t B, int64_t T, int64_t C) {
    return B * ((T + WKV_SAVED_STATE_TOKENS - 1) / WKV_SAVED_STATE_TOKENS) * 2 * C * 4;
}

// r == nullptr: plain forward; else the gated form (y = sigmoid(r) * wkv).
// states != nullptr (chained path, empty history): the carries are saved too.
int forward_impl(int64_t B, int64_t T, int64_t C, int dtype, int path, const float* w,
                 const float* u, const void* k, const void* v, const void* r, void* y,
                 const float* a_in, const float* b_in, const float* p_in, float* a_out,
                 float* b_out, float* p_out, void* workspace, size_t workspace_bytes, void* stream,
                 bool gated, float* states = nullptr) {
    if (dtype != WKV_F32 && dtype != WKV_BF16) return fail(WKV_ERR_DTYPE, "unknown dtype %d", dtype);
    if (path != WKV_PATH_AUTO && path != WKV_PATH_SERIAL && path != WKV_PATH_CHUNKED &&
        path != WKV_PATH_CHAINED)
        return fail(WKV_ERR_ARG, "unknown path %d", path);
    if (B < 1 || C < 1 || T < 0)
        return fail(WKV_ERR_SHAPE, "need B >= 1, T >= 0, C >= 1 (got B=%lld T=%lld C=%lld)",
                    (long long)B, (long long)T, (long long)C);
    int64_t n = 0;
    if (!mul3(B, T, C, &n) || !mul3(n, 4, 1, &n) || !mul3(B, C, 12, &n))
        return fail(WKV_ERR_SHAPE, "B*T*C too large");
    // every kernel addresses the tokens of one block (at most 32 rows) from
    // a 64-bit base with 32-bit byte offsets
    if (double(C) * double(esize(dtype)) * 33.0 + 512.0 > 4294967295.0)
        return fail(WKV_ERR_SHAPE, "C too large for 32-bit offsets within a block of tokens");
    const bool has_in = a_in || b_in || p_in;
    const bool has_out = a_out || b_out || p_out;
    if (has_in && !(a_in && b_in && p_in)) return fail(WKV_ERR_NULL, "a_in, b_in, p_in: all or none");
    if (has_out && !(a_out && b_out && p_out))
        return fail(WKV_ERR_NULL, "a_out, b_out, p_out: all or none");
    if (!w || !u) return fail(WKV_ERR_NULL, "w and u are required");
    if (T > 0 && (!k || !v || !y)) return fail(WKV_ERR_NULL, "k, v and y are required when T > 0");
    if (gated && T > 0 && !r) return fail(WKV_ERR_NULL, "r is required when T > 0");

    const int64_t io_bytes = B * T * C * int64_t(esize(dtype));
    const int64_t st_bytes = B * C * 4;
    const Range r_in[] = {rng("a_in", a_in, st_bytes), rng("b_in", b_in, st_bytes),
                          rng("p_in", p_in, st_bytes), rng("k", k, io_bytes),
                          rng("v", v, io_bytes), rng("w", w, C * 4), rng("u", u, C * 4),
                          rng("r", gated ? r : nullptr, io_bytes)};
    const Range r_y = rng("y", y, io_bytes);
    for (const Range& ri : r_in)
        if (overlap(r_y, ri)) return fail(WKV_ERR_ALIAS, "y overlaps %s", ri.name);
    const Range r_out[] = {rng("a_out", a_out, st_bytes), rng("b_out", b_out, st_bytes),
                           rng("p_out", p_out, st_bytes)};
    if (int rc = check_state_aliasing(r_out, 3, r_in, 8, true)) return rc;
    for (const Range& ro : r_out)
        if (overlap(ro, r_y)) return fail(WKV_ERR_ALIAS, "%s overlaps y", ro.name);
    if (states != nullptr) {
        const Range r_st = rng("states", states, saved_state_bytes(B, T, C));
        for (const Range& ri : r_in)
            if (overlap(r_st, ri)) return fail(WKV_ERR_ALIAS, "states overlaps %s", ri.name);
        for (const Range& ro : r_out)
            if (overlap(r_st, ro)) return fail(WKV_ERR_ALIAS, "states overlaps %s", ro.name);
        if (overlap(r_st, r_y)) return fail(WKV_ERR_ALIAS, "states overlaps y");
        if (!aligned(states, 8)) return fail(WKV_ERR_ARG, "states must be 8-byte aligned");
    }

    wkv::ForwardProblem pr;
    pr.B = B;
    pr.T = T;
    pr.C = C;
    pr.dtype = dtype;
    pr.vec = wkv::pick_forward_vec(C, dtype, aligned(k, 4) && aligned(v, 4) && aligned(y, 4) &&
                                                  (!gated || aligned(r, 4)));
    pr.w = w;
    pr.u = u;
    pr.k = k;
    pr.v = v;
    pr.y = y;
    pr.a_in = a_in;
    pr.b_in = b_in;
    pr.p_in = p_in;
    pr.a_out = a_out;
    pr.b_out = b_out;
    pr.p_out = p_out;
    pr.r = gated ? r : nullptr;
    pr.states = states;
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (T == 0) {
        if (!has_out) return ok();
        hipError_t e = wkv::launch_state_passthrough(pr, s);
        return e == hipSuccess ? ok() : hip_fail(e, "state copy launch");
    }
    if (path == WKV_PATH_AUTO) path = wkv::choose_forward_path(pr, wkv::device_cu_count());
    if (path == WKV_PATH_CHUNKED) {
        const wkv::ChunkPlan pl = wkv::plan_chunked(B, T, C, pr.vec);
        if (double(pl.ngroups) * double(pl.tiles_per_group) > 2147483647.0)
            return fail(WKV_ERR_SHAPE, "too many tiles for one launch");
        const size_t need = wkv::forward_workspace_bytes(B, T, C, dtype, WKV_PATH_CHUNKED);
        if (workspace == nullptr || workspace_bytes < need)
            return fail(WKV_ERR_WORKSPACE, "chunked path needs %zu workspace bytes, got %zu", need,
                        workspace ? workspace_bytes : size_t(0));
        if (!aligned(workspace, 256)) return fail(WKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        const Range r_ws = rng("workspace", workspace, int64_t(need));
        for (const Range& ri : r_in)
            if (overlap(r_ws, ri)) return fail(WKV_ERR_ALIAS, "workspace overlaps %s", ri.name);
        for (const Range& ro : r_out)
            if (overlap(r_ws, ro)) return fail(WKV_ERR_ALIAS, "workspace overlaps %s", ro.name);
        if (overlap(r_ws, r_y)) return fail(WKV_ERR_ALIAS, "workspace overlaps y");
        hipError_t e = wkv::launch_forward_chunked(pr, workspace, s);
        return e == hipSuccess ? ok() : hip_fail(e, "chunked forward launch");
    }
    const int64_t cg = 64 * pr.vec;
    if (double(B) * double((C + cg - 1) / cg) > 2147483647.0)
        return fail(WKV_ERR_SHAPE, "too many column groups for one launch");
    if (path == WKV_PATH_CHAINED) {
        hipError_t e = wkv::launch_forward_chained(pr, s);
        return e == hipSuccess ? ok() : hip_fail(e, "chained forward launch");
    }
    hipError_t e = wkv::launch_forward_serial(pr, s);
    return e == hipSuccess ? ok() : hip_fail(e, "serial forward launch");
}

std::atomic<int> g_cus[64];

}  // namespace

namespace wkv_detail {
// Error reporting for the other host files of the library.
int fail_status(int status, const char* msg) { return fail(status, "%s", msg); }
int ok_status() { return ok(); }
}  // namespace wkv_detail

namespace wkv {
int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}
}  // namespace wkv

extern "C" {

int wkv_abi_version(void) { return WKV_ABI_VERSION; }

int wkv_bounded_wait_failures(uint64_t* count) {
    if (!count) return fail(WKV_ERR_NULL, "count is required");
    uint64_t a = 0, b = 0;
    hipError_t e = wkv::read_chunk_wait_failures(&a);
    if (e != hipSuccess) return hip_fail(e, "reading the look-back failure count");
    e = wkv::read_ring_wait_failures(&b);
    if (e != hipSuccess) return hip_fail(e, "reading the ring failure count");
    *count = a + b;
    return ok();
}

const char* wkv_status_string(int status) {
    switch (status) {
        case WKV_OK: return "ok";
        case WKV_ERR_NULL: return "a required pointer is NULL";
        case WKV_ERR_SHAPE: return "invalid or too large shape";
        case WKV_ERR_DTYPE: return "unknown dtype";
        case WKV_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case WKV_ERR_ALIAS: return "an output overlaps an input it may not overlap";
        case WKV_ERR_HIP: return "HIP runtime error";
        case WKV_ERR_UNSUPPORTED: return "unsupported option";
        case WKV_ERR_ARG: return "argument out of range";
        default: return "unknown status";
    }
}

const char* wkv_last_error(void) { return g_last_error.c_str(); }

size_t wkv_forward_workspace_size_path(int64_t B, int64_t T, int64_t C, int dtype, int path) {
    if (B < 1 || C < 1 || T < 0) return 0;
    if (dtype != WKV_F32 && dtype != WKV_BF16) return 0;
    int64_t n = 0;
    if (!mul3(B, T, C, &n)) return 0;
    if (path == WKV_PATH_AUTO) {
        wkv::ForwardProblem pr{};
        pr.B = B;
        pr.T = T;
        pr.C = C;
        pr.dtype = dtype;
        pr.vec = wkv::pick_forward_vec(C, dtype, true);
        path = wkv::choose_forward_path(pr, wkv::device_cu_count());
        // the chosen vec can be 1 for misaligned pointers: cover both
        if (path != WKV_PATH_CHUNKED) {
            pr.vec = 1;
            path = wkv::choose_forward_path(pr, wkv::device_cu_count());
        }
    }
    return wkv::forward_workspace_bytes(B, T, C, dtype, path);
}

int wkv_forward_auto_path(int64_t B, int64_t T, int64_t C, int dtype) {
    if (B < 1 || C < 1 || T < 0) return fail(WKV_ERR_SHAPE, "need B >= 1, T >= 0, C >= 1");
    if (dtype != WKV_F32 && dtype != WKV_BF16) return fail(WKV_ERR_DTYPE, "unknown dtype %d", dtype);
    int64_t n = 0;
    if (!mul3(B, T, C, &n)) return fail(WKV_ERR_SHAPE, "B*T*C too large");
    wkv::ForwardProblem pr{};
    pr.B = B;
    pr.T = T;
    pr.C = C;
    pr.dtype = dtype;
    pr.vec = wkv::pick_forward_vec(C, dtype, true);
    return wkv::choose_forward_path(pr, wkv::device_cu_count());
}

size_t wkv_forward_workspace_size(int64_t B, int64_t T, int64_t C, int dtype) {
    return wkv_forward_workspace_size_path(B, T, C, dtype, WKV_PATH_AUTO);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch memory of wkv_forward_noalloc: a fixed device array, one copy per
// device, that stands in for the chunked path's workspace.  Host code never
// uses the array's name as an address (it is a host-side stand-in): the
// device address of this device's copy comes from hipGetSymbolAddress, once
// per device, and only that pointer is handed to the kernels.
// ---------------------------------------------------------------------------

static __device__ __align__(256) unsigned char scratch[WKV_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<void*> g_scratch_ptr[64];
std::mutex g_scratch_mutex;

int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(WKV_ERR_UNSUPPORTED, "device index %d out of range", dev);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
            if (p == nullptr) return fail(WKV_ERR_HIP, "hipGetSymbolAddress gave no scratch address");
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return WKV_OK;
}

}  // namespace

extern "C" {

int wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, int dtype, const float* w, const float* u,
                        const void* k, const void* v, void* y, const float* a_in, const float* b_in,
                        const float* p_in, float* a_out, float* b_out, float* p_out, void* stream) {
    // the sizes are validated in full by forward_impl; here only the scratch need
    const size_t need = wkv_forward_workspace_size(B, T, C, dtype);
    if (need > size_t(WKV_NOALLOC_SCRATCH_BYTES))
        return fail(WKV_ERR_WORKSPACE,
                    "these sizes need %zu bytes of scratch; wkv_forward_noalloc has %zu "
                    "(use wkv_forward with a workspace)",
                    need, size_t(WKV_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    if (need > 0)
        if (int rc = scratch_address(&ws)) return rc;
    return forward_impl(B, T, C, dtype, WKV_PATH_AUTO, w, u, k, v, nullptr, y, a_in, b_in, p_in,
                        a_out, b_out, p_out, ws, need > 0 ? size_t(WKV_NOALLOC_SCRATCH_BYTES) : 0,
                        stream, false);
}

int wkv_forward(int64_t B, int64_t T, int64_t C, int dtype, const float* w, const float* u,
                const void* k, const void* v, void* y, const float* a_in, const float* b_in,
                const float* p_in, float* a_out, float* b_out, float* p_out, void* workspace,
                size_t workspace_bytes, void* stream) {
    return forward_impl(B, T, C, dtype, WKV_PATH_AUTO, w, u, k, v, nullptr, y, a_in, b_in, p_in,
                        a_out, b_out, p_out, workspace, workspace_bytes, stream, false);
}

int wkv_forward_path(int64_t B, int64_t T, int64_t C, int dtype, int path, const float* w,
                     const float* u, const void* k, const void* v, void* y, const float* a_in,
                     const float* b_in, const float* p_in, float* a_out, float* b_out,
                     float* p_out, void* workspace, size_t workspace_bytes, void* stream) {
    return forward_impl(B, T, C, dtype, path, w, u, k, v, nullptr, y, a_in, b_in, p_in, a_out, b_out,
                        p_out, workspace, workspace_bytes, stream, false);
}

int wkv_forward_gated(int64_t B, int64_t T, int64_t C, int dtype, int path, const float* w,
                      const float* u, const void* k, const void* v, const void* r, void* o,
                      const float* a_in, const float* b_in, const float* p_in, float* a_out,
                      float* b_out, float* p_out, void* workspace, size_t workspace_bytes,
                      void* stream) {
    return forward_impl(B, T, C, dtype, path, w, u, k, v, r, o, a_in, b_in, p_in, a_out, b_out,
                        p_out, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

namespace {
// r == nullptr and !gated: plain step; gated: y = sigmoid(r) * wkv.
int step_impl(int64_t L, int64_t S, int64_t C, int dtype, const float* w, const float* u,
              const void* k, const void* v, const void* r, void* y, const float* a_in,
              const float* b_in, const float* p_in, float* a_out, float* b_out, float* p_out,
              void* stream, bool gated) {
    if (dtype != WKV_F32 && dtype != WKV_BF16) return fail(WKV_ERR_DTYPE, "unknown dtype %d", dtype);
    if (L < 1 || S < 1 || C < 1)
        return fail(WKV_ERR_SHAPE, "need L, S, C >= 1 (got L=%lld S=%lld C=%lld)", (long long)L,
                    (long long)S, (long long)C);
    int64_t n = 0;
    if (!mul3(L, S, C, &n) || !mul3(n, 4, 1, &n)) return fail(WKV_ERR_SHAPE, "L*S*C too large");
    n = L * S * C;
    if (!w || !u || !k || !v || !y || !a_in || !b_in || !p_in || !a_out || !b_out || !p_out)
        return fail(WKV_ERR_NULL, "every wkv_step array is required");
    if (gated && !r) return fail(WKV_ERR_NULL, "r is required");
    const int64_t io = n * int64_t(esize(dtype));
    const Range r_in[] = {rng("a_in", a_in, n * 4), rng("b_in", b_in, n * 4), rng("p_in", p_in, n * 4),
                          rng("k", k, io), rng("v", v, io), rng("w", w, L * C * 4),
                          rng("u", u, L * C * 4), rng("r", gated ? r : nullptr, io)};
    const Range r_y = rng("y", y, io);
    for (const Range& ri : r_in)
        if (overlap(r_y, ri)) return fail(WKV_ERR_ALIAS, "y overlaps %s", ri.name);
    const Range r_out[] = {rng("a_out", a_out, n * 4), rng("b_out", b_out, n * 4),
                           rng("p_out", p_out, n * 4)};
    if (int rc = check_state_aliasing(r_out, 3, r_in, 8, true)) return rc;
    for (const Range& ro : r_out)
        if (overlap(ro, r_y)) return fail(WKV_ERR_ALIAS, "%s overlaps y", ro.name);
    if (double(n) / 256.0 > 2147483647.0) return fail(WKV_ERR_SHAPE, "too many elements for one launch");

    wkv::StepProblem pr;
    pr.L = L;
    pr.S = S;
    pr.C = C;
    pr.dtype = dtype;
    const uintptr_t io_align = dtype == WKV_BF16 ? 8 : 16;
    const bool al = aligned(k, io_align) && aligned(v, io_align) && aligned(y, io_align) &&
                    (!gated || aligned(r, io_align)) &&
                    aligned(a_in, 16) && aligned(b_in, 16) && aligned(p_in, 16) &&
                    aligned(a_out, 16) && aligned(b_out, 16) && aligned(p_out, 16);
    pr.vec = (C % 4 == 0 && al) ? 4 : 1;
    pr.w = w;
    pr.u = u;
    pr.k = k;
    pr.v = v;
    pr.y = y;
    pr.a_in = a_in;
    pr.b_in = b_in;
    pr.p_in = p_in;
    pr.a_out = a_out;
    pr.b_out = b_out;
    pr.p_out = p_out;
    pr.r = gated ? r : nullptr;
    hipError_t e = wkv::launch_step(pr, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "step launch");
}
}  // namespace

extern "C" {

int wkv_step(int64_t L, int64_t S, int64_t C, int dtype, const float* w, const float* u,
             const void* k, const void* v, void* y, const float* a_in, const float* b_in,
             const float* p_in, float* a_out, float* b_out, float* p_out, void* stream) {
    return step_impl(L, S, C, dtype, w, u, k, v, nullptr, y, a_in, b_in, p_in, a_out, b_out, p_out,
                     stream, false);
}

int wkv_step_gated(int64_t L, int64_t S, int64_t C, int dtype, const float* w, const float* u,
                   const void* k, const void* v, const void* r, void* y, const float* a_in,
                   const float* b_in, const float* p_in, float* a_out, float* b_out, float* p_out,
                   void* stream) {
    return step_impl(L, S, C, dtype, w, u, k, v, r, y, a_in, b_in, p_in, a_out, b_out, p_out,
                     stream, true);
}

size_t wkv_backward_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 1 || C < 1 || T < 0) return 0;
    int64_t n = 0;
    if (!mul3(B, T, C, &n) || !mul3(n, 8, 1, &n)) return 0;
    return wkv::backward_workspace_bytes(B, T, C, false);
}

}  // extern "C"

namespace {
// states != nullptr: the saved checkpoints of wkv_forward_save.
int backward_impl(int64_t B, int64_t T, int64_t C, int dtype, const float* w, const float* u,
                  const void* k, const void* v, const void* gy, const float* states, void* gk,
                  void* gv, float* gw, float* gu, void* workspace, size_t workspace_bytes,
                  void* stream) {
    if (dtype != WKV_F32 && dtype != WKV_BF16) return fail(WKV_ERR_DTYPE, "unknown dtype %d", dtype);
    if (B < 1 || C < 1 || T < 0)
        return fail(WKV_ERR_SHAPE, "need B >= 1, T >= 0, C >= 1 (got B=%lld T=%lld C=%lld)",
                    (long long)B, (long long)T, (long long)C);
    int64_t n = 0;
    if (!mul3(B, T, C, &n) || !mul3(n, 8, 1, &n) || !mul3(B, C, 8, &n))
        return fail(WKV_ERR_SHAPE, "B*T*C too large");
    n = B * T * C;
    if (!w || !u || !gw || !gu) return fail(WKV_ERR_NULL, "w, u, gw and gu are required");
    if (T > 0 && (!k || !v || !gy || !gk || !gv))
        return fail(WKV_ERR_NULL, "k, v, gy, gk and gv are required when T > 0");
    if (double(B) * double((C + 63) / 64) > 2147483647.0)
        return fail(WKV_ERR_SHAPE, "too many column groups for one launch");
    if (double(C) * 4.0 * 17.0 > 4294967295.0)
        return fail(WKV_ERR_SHAPE, "C too large for 32-bit offsets within a sub-chunk");
    const int64_t io = n * int64_t(esize(dtype));
    const bool saved = states != nullptr;
    if (saved && T > 0 && !aligned(states, 8)) return fail(WKV_ERR_ARG, "states must be 8-byte aligned");
    const Range r_in[] = {rng("k", k, io), rng("v", v, io), rng("gy", gy, io), rng("w", w, C * 4),
                          rng("u", u, C * 4),
                          rng("states", T > 0 ? states : nullptr, saved_state_bytes(B, T, C))};
    const size_t need = T > 0 ? wkv::backward_workspace_bytes(B, T, C, saved) : 0;
    const Range r_out[] = {rng("gk", gk, io), rng("gv", gv, io), rng("gw", gw, C * 4),
                           rng("gu", gu, C * 4), rng("workspace", T > 0 ? workspace : nullptr, int64_t(need))};
    for (int i = 0; i < 5; i++) {
        for (const Range& r : r_in)
            if (overlap(r_out[i], r)) return fail(WKV_ERR_ALIAS, "%s overlaps %s", r_out[i].name, r.name);
        for (int j = 0; j < i; j++)
            if (overlap(r_out[i], r_out[j]))
                return fail(WKV_ERR_ALIAS, "%s overlaps %s", r_out[i].name, r_out[j].name);
    }
    if (T > 0) {
        if (workspace == nullptr || workspace_bytes < need)
            return fail(WKV_ERR_WORKSPACE, "backward needs %zu workspace bytes, got %zu", need,
                        workspace ? workspace_bytes : size_t(0));
        if (!aligned(workspace, 256)) return fail(WKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    wkv::BackwardProblem pr;
    pr.B = B;
    pr.T = T;
    pr.C = C;
    pr.dtype = dtype;
    pr.w = w;
    pr.u = u;
    pr.k = k;
    pr.v = v;
    pr.gy = gy;
    pr.gk = gk;
    pr.gv = gv;
    pr.gw = gw;
    pr.gu = gu;
    pr.saved = saved ? states : nullptr;
    pr.vec = wkv::backward_vec(C, dtype, aligned(k, 4) && aligned(v, 4) && aligned(gy, 4) &&
                                             aligned(gk, 4) && aligned(gv, 4));
    hipError_t e = wkv::launch_backward(pr, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "backward launch");
}
}  // namespace

extern "C" {

int wkv_backward(int64_t B, int64_t T, int64_t C, int dtype, const float* w, const float* u,
                 const void* k, const void* v, const void* gy, void* gk, void* gv, float* gw,
                 float* gu, void* workspace, size_t workspace_bytes, void* stream) {
    return backward_impl(B, T, C, dtype, w, u, k, v, gy, nullptr, gk, gv, gw, gu, workspace,
                         workspace_bytes, stream);
}

size_t wkv_saved_states_bytes(int64_t B, int64_t T, int64_t C) {
    if (B < 1 || C < 1 || T < 0) return 0;
    int64_t n = 0;
    if (!mul3(B, T, C, &n) || !mul3(n, 8, 1, &n)) return 0;
    return size_t(saved_state_bytes(B, T, C));
}

int wkv_forward_save(int64_t B, int64_t T, int64_t C, int dtype, const float* w, const float* u,
                     const void* k, const void* v, void* y, float* states, void* stream) {
    if (T > 0 && states == nullptr) return fail(WKV_ERR_NULL, "states is required when T > 0");
    return forward_impl(B, T, C, dtype, WKV_PATH_CHAINED, w, u, k, v, nullptr, y, nullptr, nullptr,
                        nullptr, nullptr, nullptr, nullptr, nullptr, 0, stream, false,
                        T > 0 ? states : nullptr);
}

size_t wkv_backward_saved_workspace_size(int64_t B, int64_t C) {
    if (B < 1 || C < 1) return 0;
    int64_t n = 0;
    if (!mul3(B, C, 8, &n)) return 0;
    return wkv::backward_workspace_bytes(B, 1, C, true);
}

int wkv_backward_saved(int64_t B, int64_t T, int64_t C, int dtype, const float* w, const float* u,
                       const void* k, const void* v, const void* gy, const float* states, void* gk,
                       void* gv, float* gw, float* gu, void* workspace, size_t workspace_bytes,
                       void* stream) {
    if (T > 0 && states == nullptr) return fail(WKV_ERR_NULL, "states is required when T > 0");
    return backward_impl(B, T, C, dtype, w, u, k, v, gy, states, gk, gv, gw, gu, workspace,
                         workspace_bytes, stream);
}

int wkv_token_shift(int64_t B, int64_t T, int64_t C, int dtype, const void* x, const void* x_prev,
                    const float* mu_r, const float* mu_k, const float* mu_v, void* xr, void* xk,
                    void* xv, void* x_last, void* stream) {
    if (dtype != WKV_F32 && dtype != WKV_BF16) return fail(WKV_ERR_DTYPE, "unknown dtype %d", dtype);
    if (B < 1 || C < 1 || T < 0)
        return fail(WKV_ERR_SHAPE, "need B >= 1, T >= 0, C >= 1 (got B=%lld T=%lld C=%lld)",
                    (long long)B, (long long)T, (long long)C);
    int64_t n = 0;
    if (!mul3(B, T, C, &n) || !mul3(n, 4, 1, &n)) return fail(WKV_ERR_SHAPE, "B*T*C too large");
    n = B * T * C;
    if (!mu_r || !mu_k || !mu_v) return fail(WKV_ERR_NULL, "mu_r, mu_k, mu_v are required");
    if (T > 0 && (!x || !xr || !xk || !xv)) return fail(WKV_ERR_NULL, "x, xr, xk, xv are required");
    const int64_t es = int64_t(esize(dtype));
    const Range r_in[] = {rng("x", x, n * es), rng("x_prev", x_prev, B * C * es),
                          rng("mu_r", mu_r, C * 4), rng("mu_k", mu_k, C * 4), rng("mu_v", mu_v, C * 4)};
    const Range r_out[] = {rng("xr", xr, n * es), rng("xk", xk, n * es), rng("xv", xv, n * es),
                           rng("x_last", x_last, B * C * es)};
    for (int i = 0; i < 4; i++) {
        for (const Range& r : r_in)
            if (overlap(r_out[i], r)) return fail(WKV_ERR_ALIAS, "%s overlaps %s", r_out[i].name, r.name);
        for (int j = 0; j < i; j++)
            if (overlap(r_out[i], r_out[j]))
                return fail(WKV_ERR_ALIAS, "%s overlaps %s", r_out[i].name, r_out[j].name);
    }
    // the widest lane access (16 bytes at most) that C and every array allow
    int vec = 1;
    for (int cand : {8, 4, 2}) {
        const uintptr_t a = uintptr_t(cand) * uintptr_t(es);
        if (a <= 16 && C % cand == 0 && aligned(x, a) && aligned(xr, a) && aligned(xk, a) &&
            aligned(xv, a) && aligned(x_prev, a) && aligned(x_last, a)) {
            vec = cand;
            break;
        }
    }
    if (double(B) * double((T + wkv::kShiftTokens - 1) / wkv::kShiftTokens) * double(C / vec) / 256.0 >
        2147483647.0)
        return fail(WKV_ERR_SHAPE, "too many elements for one launch");
    wkv::ShiftProblem pr;
    pr.B = B;
    pr.T = T;
    pr.C = C;
    pr.dtype = dtype;
    pr.vec = vec;
    pr.x = x;
    pr.x_prev = x_prev;
    pr.mu_r = mu_r;
    pr.mu_k = mu_k;
    pr.mu_v = mu_v;
    pr.xr = xr;
    pr.xk = xk;
    pr.xv = xv;
    pr.x_last = x_last;
    hipError_t e = wkv::launch_token_shift(pr, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "token shift launch");
}


}  // extern "C"

namespace {

// Shared checks of the matrix-state calls: nrows token rows of C = 64 H
// channels, z per token (dtype, like r) or per channel (fp32, zrows x C), a
// state of nheads 64 x 64 fp32 blocks.
int mat_check(int dtype, int64_t nrows, int64_t H, const void* r, const void* k, const void* v,
              const void* z, int z_mode, int64_t zrows, const float* s_in, const float* s_out,
              int64_t nheads, const void* y, bool same_state_ok) {
    if (dtype != WKV_F32 && dtype != WKV_BF16) return fail(WKV_ERR_DTYPE, "unknown dtype %d", dtype);
    if (z_mode != WKV_MAT_DECAY_PER_CHANNEL && z_mode != WKV_MAT_DECAY_PER_TOKEN)
        return fail(WKV_ERR_ARG, "unknown z_mode %d", z_mode);
    const int64_t C = H * WKV_MAT_HEAD_DIM;
    const int64_t io = nrows * C * int64_t(esize(dtype));
    const int64_t st = nheads * WKV_MAT_HEAD_DIM * WKV_MAT_HEAD_DIM * 4;
    const int64_t zb = z_mode == WKV_MAT_DECAY_PER_TOKEN ? io : zrows * C * 4;
    const uintptr_t al = dtype == WKV_BF16 ? 8 : 16;
    if (nrows > 0) {
        if (!r || !k || !v || !z || !y) return fail(WKV_ERR_NULL, "r, k, v, z and y are required");
        if (!aligned(r, al) || !aligned(k, al) || !aligned(v, al) || !aligned(y, al) ||
            (z_mode == WKV_MAT_DECAY_PER_TOKEN && !aligned(z, al)) || !aligned(z, 4))
            return fail(WKV_ERR_ARG, "r, k, v, z, y must be %d-byte aligned", int(al));
    }
    if ((s_in && !aligned(s_in, 4)) || (s_out && !aligned(s_out, 4)))
        return fail(WKV_ERR_ARG, "the state arrays must be 4-byte aligned");
    const Range ins[] = {rng("s_in", s_in, st), rng("r", r, io), rng("k", k, io), rng("v", v, io),
                         rng("z", z, zb)};
    const Range ry = rng("y", y, io);
    for (const Range& ri : ins)
        if (overlap(ry, ri)) return fail(WKV_ERR_ALIAS, "y overlaps %s", ri.name);
    const Range so[] = {rng("s_out", s_out, st)};
    if (int rc = check_state_aliasing(so, 1, ins, 5, same_state_ok)) return rc;
    if (overlap(so[0], ry)) return fail(WKV_ERR_ALIAS, "s_out overlaps y");
    return WKV_OK;
}

}  // namespace

extern "C" {

int wkv_mat_forward_path(int64_t B, int64_t T, int64_t H, int dtype, int path, const void* r,
                         const void* k, const void* v, const void* z, int z_mode,
                         const float* s_in, float* s_out, void* y, void* stream) {
    if (B < 1 || H < 1 || T < 0)
        return fail(WKV_ERR_SHAPE, "need B >= 1, T >= 0, H >= 1 (got B=%lld T=%lld H=%lld)",
                    (long long)B, (long long)T, (long long)H);
    if (path != WKV_MAT_PATH_AUTO && path != WKV_MAT_PATH_CHUNKED && path != WKV_MAT_PATH_TOKENWISE)
        return fail(WKV_ERR_ARG, "unknown path %d", path);
    if (path == WKV_MAT_PATH_CHUNKED && dtype == WKV_F32)
        return fail(WKV_ERR_UNSUPPORTED, "the chunked matrix-core path takes bf16 storage only");
    int64_t n = 0;
    if (!mul3(B, T, H * WKV_MAT_HEAD_DIM, &n) || !mul3(n, 4, 1, &n) ||
        !mul3(B * H, WKV_MAT_HEAD_DIM * WKV_MAT_HEAD_DIM, 4, &n))
        return fail(WKV_ERR_SHAPE, "sizes too large");
    if (B * H > 2147483647) return fail(WKV_ERR_SHAPE, "B*H too large for one launch");
    // rows of a chunk of tokens are addressed with 32-bit byte offsets
    if (double(H) * WKV_MAT_HEAD_DIM * 4.0 * 17.0 > 4294967295.0)
        return fail(WKV_ERR_SHAPE, "H too large for 32-bit offsets within a chunk of tokens");
    if (int rc = mat_check(dtype, B * T, H, r, k, v, z, z_mode, 1, s_in, s_out, B * H, y, true))
        return rc;
    wkv::MatProblem pr;
    pr.B = B;
    pr.T = T;
    pr.H = H;
    pr.dtype = dtype;
    pr.r = r;
    pr.k = k;
    pr.v = v;
    pr.z = z;
    pr.z_per_token = z_mode == WKV_MAT_DECAY_PER_TOKEN;
    pr.s_in = s_in;
    pr.s_out = s_out;
    pr.y = y;
    pr.path = path == WKV_MAT_PATH_TOKENWISE ? 1 : 0;
    if (T == 0 && s_out == nullptr) return ok();
    hipError_t e = wkv::launch_mat_forward(pr, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "matrix-state forward launch");
}

int wkv_mat_forward(int64_t B, int64_t T, int64_t H, int dtype, const void* r, const void* k,
                    const void* v, const void* z, int z_mode, const float* s_in, float* s_out,
                    void* y, void* stream) {
    return wkv_mat_forward_path(B, T, H, dtype, WKV_MAT_PATH_AUTO, r, k, v, z, z_mode, s_in, s_out,
                                y, stream);
}

int wkv_mat_step(int64_t L, int64_t S, int64_t H, int dtype, const void* r, const void* k,
                 const void* v, const void* z, int z_mode, const float* s_in, float* s_out,
                 void* y, void* stream) {
    if (L < 1 || S < 1 || H < 1)
        return fail(WKV_ERR_SHAPE, "need L, S, H >= 1 (got L=%lld S=%lld H=%lld)", (long long)L,
                    (long long)S, (long long)H);
    int64_t n = 0;
    if (!mul3(L, S, H * WKV_MAT_HEAD_DIM * WKV_MAT_HEAD_DIM, &n) || !mul3(n, 4, 1, &n))
        return fail(WKV_ERR_SHAPE, "sizes too large");
    if ((L * S * H + 3) / 4 > 2147483647) return fail(WKV_ERR_SHAPE, "too many heads for one launch");
    if (!s_in || !s_out) return fail(WKV_ERR_NULL, "s_in and s_out are required");
    if (!aligned(s_in, 16) || !aligned(s_out, 16))
        return fail(WKV_ERR_ARG, "the decode state arrays must be 16-byte aligned");
    if (int rc = mat_check(dtype, L * S, H, r, k, v, z, z_mode, L, s_in, s_out, L * S * H, y, true))
        return rc;
    wkv::MatStepProblem pr;
    pr.L = L;
    pr.S = S;
    pr.H = H;
    pr.dtype = dtype;
    pr.r = r;
    pr.k = k;
    pr.v = v;
    pr.z = z;
    pr.z_per_token = z_mode == WKV_MAT_DECAY_PER_TOKEN;
    pr.s_in = s_in;
    pr.s_out = s_out;
    pr.y = y;
    hipError_t e = wkv::launch_mat_step(pr, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "matrix-state step launch");
}

}  // extern "C"
