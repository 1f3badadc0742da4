// wkv_forward kernels: the training/prefill form over [B,T,C].
//
// Three execution paths compute the same recurrence ([tm-math] = aicassindra.com
// tm_rwkv_math, "Why it collapses into a recurrence": a scan over time that
// parallelises across batch and channels; [vanos] = vanos001.github.io rwkv,
// "The WKV Operator": a serial per-position scan or a chunked parallel form).
// A column group is 64 lanes x VEC adjacent channels of one batch row.
//
// serial   One wave per column group scans all of T with the state in
//          registers.  Used when the column groups alone give every SIMD
//          several waves.
//
// chained  One workgroup of up to 16 waves per column group.  Its tokens are
//          cut into sub-chunks that the waves take round-robin; each wave
//          loads a sub-chunk into registers, folds it into a partial state,
//          receives the carry from the previous sub-chunk's wave through LDS,
//          hands carry (+) partial to the next one and re-runs its tokens to
//          write y.  k, v are read once, no workspace, timing-independent
//          results.  Used when there are about as many column groups as CUs.
//
// chunked  One workgroup per tile = (column group, NW*L consecutive tokens);
//          wave w of the tile owns L tokens.  Partial states are combined
//          across the waves of the tile in LDS and across tiles of a column
//          group through global memory with a single-pass decoupled
//          look-back (each tile publishes its aggregate, then its inclusive
//          prefix; a successor combines aggregates backwards until it meets
//          an inclusive prefix).  k, v are read once.  Tiles are handed out in
//          (chunk, group) order by an atomic ticket, so a tile only waits for
//          tiles that already started.  Used when B*C is small.
#include "wkv_device.h"
#include "wkv_internal.h"

#include <algorithm>

namespace wkv {
namespace {

// Launch geometry (the macros exist so that tuning builds can override them).
#ifndef WKV_SERIAL_TOKENS
#define WKV_SERIAL_TOKENS 16
#endif
#ifndef WKV_CHUNK_TOKENS
#define WKV_CHUNK_TOKENS 32
#endif
#ifndef WKV_CHUNK_WAVES
#define WKV_CHUNK_WAVES 8
#endif
#ifndef WKV_CHAIN_TOKENS
#define WKV_CHAIN_TOKENS 16
#endif
#ifndef WKV_FRAME_TOKENS
#define WKV_FRAME_TOKENS 8
#endif
constexpr int kSerialWaves = 4;                  // waves per workgroup on the serial path
constexpr int kSerialTokens = WKV_SERIAL_TOKENS; // tokens loaded per batch on the serial path
constexpr int kChunkTokens = WKV_CHUNK_TOKENS;   // L: tokens per wave on the chunked path
constexpr int kChunkWaves = WKV_CHUNK_WAVES;     // NW: waves per tile
constexpr int kChunkWavesWide = 2 * kChunkWaves; // the wide tiles of plan_chunked
constexpr int kChainTokens = WKV_CHAIN_TOKENS;   // tokens per sub-chunk on the chained path
constexpr int kFrameTokens = WKV_FRAME_TOKENS;   // tokens per frame of the running maximum
constexpr uint64_t kSpinTicks = 20000000;  // 200 ms at 100 MHz

// Count of look-back waits that gave up, on this device, since the library
// was loaded (read by wkv_bounded_wait_failures()).
__device__ unsigned int g_chunk_wait_failures;

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Per-lane state of VEC channels: accumulators a, b and the exponent of the
// running maximum in anchor form, p = A - m * w (m a token count).
template <int VEC>
struct Lane {
    Chan ch[VEC];
    float a[VEC], b[VEC], A[VEC], m[VEC];
};

template <int VEC>
__device__ __forceinline__ void load_params(Lane<VEC>& s, const ForwardProblem& pr, int64_t c,
                                            bool active) {
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        const float w = active ? pr.w[c + q] : 1.0f;
        const float u = active ? pr.u[c + q] : 0.0f;
        s.ch[q] = make_chan(w, u);
    }
}

template <int VEC>
__device__ __forceinline__ void load_state(float (&a)[VEC], float (&b)[VEC], float (&A)[VEC],
                                           float (&m)[VEC], const ForwardProblem& pr, int64_t col,
                                           bool active) {
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        m[q] = 0.0f;
        if (active && pr.a_in != nullptr) {
            a[q] = pr.a_in[col + q];
            b[q] = pr.b_in[col + q];
            A[q] = clamp_empty(pr.p_in[col + q]);
        } else {
            a[q] = 0.0f;
            b[q] = 0.0f;
            A[q] = kEmptyP;
        }
    }
}

template <int VEC>
__device__ __forceinline__ void store_state(const Lane<VEC>& s, const ForwardProblem& pr, int64_t col) {
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        pr.a_out[col + q] = s.a[q];
        pr.b_out[col + q] = s.b[q];
        pr.p_out[col + q] = export_p(__builtin_fmaf(-s.m[q], s.ch[q].w, s.A[q]));
    }
}

template <int VEC>
__device__ __forceinline__ bool wave_all_fused(const Lane<VEC>& s) {
    bool f = true;
#pragma unroll
    for (int q = 0; q < VEC; q++) f = f && s.ch[q].fused;
    return __builtin_amdgcn_ballot_w64(!f) == 0;
}

// Run n tokens (n == NTOK when FULL) from the state in s, writing y.  The
// tokens are the first n of kr/vr.  The frame of the running maximum (see
// wkv_device.h, 4.) moves forward every kFrameTokens tokens, so a key enters
// its frame shifted by at most kFrameTokens * w and its rounding stays at the
// scale of the key itself.  Moving the frame rounds once; an exact anchor
// and token count are kept across blocks.
// GATED: rr holds the receptance of the same tokens and the block writes
// sigmoid(r) * y.
template <int DT, int VEC, int NTOK, bool FUSED_ONLY, bool FULL, bool GATED>
__device__ __forceinline__ void run_block(Lane<VEC>& s, const typename Io<DT, VEC>::Raw (&kr)[NTOK],
                                          const typename Io<DT, VEC>::Raw (&vr)[NTOK],
                                          const typename Io<DT, VEC>::Raw (&rr)[NTOK], rsrc_t yr_,
                                          uint32_t voff, uint32_t row_bytes, int n, bool active) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int F = kFrameTokens;
    static_assert(NTOK % F == 0, "blocks are whole frames");
    float kas[VEC];
    bool all_keep[VEC];
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        kas[q] = __builtin_fmaf(-s.m[q], s.ch[q].w, s.A[q]);
        all_keep[q] = true;
    }
#pragma unroll
    for (int i = 0; i < NTOK; i++) {
        if (FULL || i < n) {
            if (i % F == 0 && i > 0) {
#pragma unroll
                for (int q = 0; q < VEC; q++) kas[q] = __builtin_fmaf(-float(F), s.ch[q].w, kas[q]);
            }
            float kf[VEC], vf[VEC], yf[VEC], gd[VEC];
            IO::unpack(kr[i], kf);
            IO::unpack(vr[i], vf);
            if constexpr (GATED) {
                float rf[VEC];
                IO::unpack(rr[i], rf);
#pragma unroll
                for (int q = 0; q < VEC; q++) gd[q] = gate_den(rf[q]);
            }
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                bool keep;
                yf[q] = frame_token<FUSED_ONLY, GATED>(s.a[q], s.b[q], kas[q], kf[q], vf[q], s.ch[q],
                                                       float(i % F + 1), keep, GATED ? gd[q] : 1.0f);
                all_keep[q] = all_keep[q] && keep;
            }
            if (active) Buf<Raw>::template store<kStreamStore>(IO::pack(yf), yr_, voff, uint32_t(i) * row_bytes);
        }
    }
    // the last frame starts at token f0 of the block
    const int last = (FULL ? NTOK : n) - 1;
    const float since = float(last - (last / F) * F + 1);  // tokens since the last frame start
    const float nf = FULL ? float(NTOK) : float(n);
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        // a new maximum inside the block becomes the anchor, in the last frame
        s.A[q] = all_keep[q] ? s.A[q] : kas[q];
        s.m[q] = all_keep[q] ? s.m[q] + nf : since;
    }
}

// The receptance array run_block reads: rr when GATED, else any array of the
// right length (never read).
template <bool GATED, typename Raw, int N, int M>
__device__ __forceinline__ const Raw (&gated_rr(const Raw (&rr)[M], const Raw (&kr)[N]))[N] {
    if constexpr (GATED)
        return rr;
    else
        return kr;
}

// ---------------------------------------------------------------------------
// serial path
// ---------------------------------------------------------------------------

template <int DT, int VEC, bool FUSED_ONLY, bool GATED>
__device__ __forceinline__ void serial_scan(Lane<VEC>& s, const ForwardProblem& pr, const char* kbase,
                                            const char* vbase, const char* rbase, char* ybase,
                                            uint32_t voff, uint32_t row_bytes, bool active) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int U = kSerialTokens;
    const int64_t T = pr.T;
    for (int64_t t0 = 0; t0 < T; t0 += U) {
        const int n = (T - t0) < U ? int(T - t0) : U;
        const int64_t off = t0 * int64_t(row_bytes);
        const rsrc_t kr_ = make_rsrc(kbase + off);
        const rsrc_t vr_ = make_rsrc(vbase + off);
        const rsrc_t rr_ = make_rsrc((GATED ? rbase : kbase) + off);
        const rsrc_t yr_ = make_rsrc(ybase + off);
        Raw kr[U], vr[U], rr[GATED ? U : 1];
        if (n == U) {
#pragma unroll
            for (int i = 0; i < U; i++) {
                kr[i] = Buf<Raw>::load(kr_, voff, uint32_t(i) * row_bytes);
                vr[i] = Buf<Raw>::load(vr_, voff, uint32_t(i) * row_bytes);
                if constexpr (GATED) rr[i] = Buf<Raw>::load(rr_, voff, uint32_t(i) * row_bytes);
            }
            run_block<DT, VEC, U, FUSED_ONLY, true, GATED>(s, kr, vr, gated_rr<GATED>(rr, kr), yr_,
                                                           voff, row_bytes, n, active);
        } else {
#pragma unroll
            for (int i = 0; i < U; i++) {
                kr[i] = IO::zero();
                vr[i] = IO::zero();
                if constexpr (GATED) rr[i] = IO::zero();
                if (i < n) {
                    kr[i] = Buf<Raw>::load(kr_, voff, uint32_t(i) * row_bytes);
                    vr[i] = Buf<Raw>::load(vr_, voff, uint32_t(i) * row_bytes);
                    if constexpr (GATED) rr[i] = Buf<Raw>::load(rr_, voff, uint32_t(i) * row_bytes);
                }
            }
            run_block<DT, VEC, U, FUSED_ONLY, false, GATED>(s, kr, vr, gated_rr<GATED>(rr, kr), yr_,
                                                            voff, row_bytes, n, active);
        }
    }
}

template <int DT, int VEC, bool GATED>
__global__ __launch_bounds__(kSerialWaves * 64) void forward_serial_kernel(ForwardProblem pr,
                                                                           int64_t ngroups,
                                                                           int64_t gpr) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    const int64_t g = int64_t(blockIdx.x) * kSerialWaves + wave_id();
    if (g >= ngroups) return;
    const int lane = lane_id();
    const int64_t bb = g / gpr;
    const int64_t c0 = (g - bb * gpr) * (64 * VEC);
    const int64_t c = c0 + int64_t(lane) * VEC;
    const bool active = c < pr.C;
    constexpr int64_t es = sizeof(Raw) / VEC;
    const uint32_t row_bytes = uint32_t(pr.C * es);
    // lanes past C read lane 0's words (in bounds) and never store
    const uint32_t voff = active ? uint32_t(lane) * uint32_t(sizeof(Raw)) : 0u;
    const int64_t base = (bb * pr.T * pr.C + c0) * es;

    Lane<VEC> s;
    load_params(s, pr, c, active);
    load_state(s.a, s.b, s.A, s.m, pr, bb * pr.C + c, active);

    const char* kbase = static_cast<const char*>(pr.k) + base;
    const char* vbase = static_cast<const char*>(pr.v) + base;
    const char* rbase = GATED ? static_cast<const char*>(pr.r) + base : nullptr;
    char* ybase = static_cast<char*>(pr.y) + base;
    if (wave_all_fused(s))
        serial_scan<DT, VEC, true, GATED>(s, pr, kbase, vbase, rbase, ybase, voff, row_bytes, active);
    else
        serial_scan<DT, VEC, false, GATED>(s, pr, kbase, vbase, rbase, ybase, voff, row_bytes, active);
    if (active && pr.a_out != nullptr) store_state(s, pr, bb * pr.C + c);
}

// ---------------------------------------------------------------------------
// chunked path
// ---------------------------------------------------------------------------

struct ChunkArgs {
    int64_t ngroups;          // column groups
    int64_t gpr;              // column groups per batch row
    int64_t tiles_per_group;  // tiles along T
    uint32_t* ticket;         // tile dispenser (zeroed before the launch)
    uint32_t* error;          // set to 1 if a look-back wait gave up
    uint64_t* flags;          // [ngroups * tiles_per_group]: status, zeroed before the launch
    float* desc;              // [ngroups * tiles_per_group][2][4][64 * VEC]
};

// Tile status.  Every flag is cleared by a kernel launched just before the
// tiles, so a launch never sees another launch's flags, also when the pair
// of launches is recorded once in a HIP graph and replayed.
enum : uint64_t { kEmpty = 0, kAggregate = 1, kInclusive = 2 };

// a partial state in anchor form, VEC channels
template <int VEC>
struct Part {
    float a[VEC], b[VEC], A[VEC], m[VEC];
    __device__ __forceinline__ void set_empty() {
#pragma unroll
        for (int q = 0; q < VEC; q++) { a[q] = 0.0f; b[q] = 0.0f; A[q] = kEmptyP; m[q] = 0.0f; }
    }
    // this <- this (+) g, g spanning n tokens
    __device__ __forceinline__ void absorb(const Part& g, float n, const Lane<VEC>& s) {
#pragma unroll
        for (int q = 0; q < VEC; q++)
            combine(a[q], b[q], A[q], m[q], g.a[q], g.b[q], g.A[q], g.m[q], n, s.ch[q].w);
    }
};

template <int VEC>
__device__ __forceinline__ float* desc_ptr(const ChunkArgs& ca, int64_t g, int64_t j, int kind) {
    return ca.desc + ((g * ca.tiles_per_group + j) * 2 + kind) * (4 * 64 * VEC);
}

template <int VEC>
__device__ __forceinline__ void publish(const ChunkArgs& ca, int64_t g, int64_t j, int kind,
                                        const Part<VEC>& x, int lane) {
    float* d = desc_ptr<VEC>(ca, g, j, kind);
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        st_agent(d + 0 * 64 * VEC + lane * VEC + q, x.a[q]);
        st_agent(d + 1 * 64 * VEC + lane * VEC + q, x.b[q]);
        st_agent(d + 2 * 64 * VEC + lane * VEC + q, x.A[q]);
        st_agent(d + 3 * 64 * VEC + lane * VEC + q, x.m[q]);
    }
    wait_all_memory();
    if (lane == 0)
        st_flag(ca.flags + g * ca.tiles_per_group + j, kind == 0 ? kAggregate : kInclusive);
}

template <int VEC>
__device__ __forceinline__ void read_desc(const ChunkArgs& ca, int64_t g, int64_t j, int kind,
                                          Part<VEC>& x, int lane) {
    const float* d = desc_ptr<VEC>(ca, g, j, kind);
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        x.a[q] = ld_agent(d + 0 * 64 * VEC + lane * VEC + q);
        x.b[q] = ld_agent(d + 1 * 64 * VEC + lane * VEC + q);
        x.A[q] = ld_agent(d + 2 * 64 * VEC + lane * VEC + q);
        x.m[q] = ld_agent(d + 3 * 64 * VEC + lane * VEC + q);
    }
}

// Exclusive prefix of tile j of group g: combine published aggregates of
// tiles j-1, j-2, ... (newest first) until an inclusive prefix is found.
template <int VEC>
__device__ void look_back(const ChunkArgs& ca, int64_t g, int64_t j, int tile_tokens,
                          const Lane<VEC>& s, Part<VEC>& x, int lane) {
    Part<VEC> sfx;  // combined aggregates of tiles jj+1 .. j-1
    sfx.set_empty();
    float span = 0.0f;
    for (int64_t jj = j - 1;; jj--) {
        const uint64_t* fp = ca.flags + g * ca.tiles_per_group + jj;
        uint64_t f = 0;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            const uint64_t raw = ld_flag(fp);
            const uint64_t seen = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(raw)))) |
                                  (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(raw >> 32)))) << 32);
            if (seen != kEmpty) { f = seen; break; }
            // bounded wait: give up after kSpinTicks of the 100 MHz real-time
            // counter, or at once when another tile already gave up
            if (__builtin_amdgcn_readfirstlane(
                    __hip_atomic_load(ca.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0)
                break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) break;
            __builtin_amdgcn_s_sleep(2);
        }
        compiler_fence();
        if (f == 0) {
            // never expected.  The kernel still terminates, and the miss is
            // made visible: the carry becomes NaN, so this tile's outputs and
            // (through its inclusive prefix) every later tile's of the column
            // group are NaN; the workspace error word and the device's
            // failure count record it.
            if (lane == 0) {
                atomicOr(ca.error, 1u);
                atomicAdd(&g_chunk_wait_failures, 1u);
            }
            const float nan = __builtin_nanf("");
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                x.a[q] = nan;
                x.b[q] = nan;
                x.A[q] = 0.0f;
                x.m[q] = 0.0f;
            }
            return;
        }
        const int kind = f == kInclusive ? 1 : 0;
        Part<VEC> d;
        read_desc<VEC>(ca, g, jj, kind, d, lane);
        d.absorb(sfx, span, s);
        if (kind == 1) {
            x = d;
            return;
        }
        sfx = d;
        span += float(tile_tokens);
    }
}

// Load this wave's n tokens of k, v (n == L when FULL) with cache policy AUX.
template <int DT, int VEC, int L, bool FULL, int AUX>
__device__ __forceinline__ void chunk_load(typename Io<DT, VEC>::Raw (&kr)[L],
                                           typename Io<DT, VEC>::Raw (&vr)[L], rsrc_t kr_,
                                           rsrc_t vr_, uint32_t voff, uint32_t row_bytes, int n) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
#pragma unroll
    for (int i = 0; i < L; i++) {
        if (FULL || i < n) {
            kr[i] = Buf<Raw>::template load<AUX>(kr_, voff + uint32_t(i) * row_bytes, 0u);
            vr[i] = Buf<Raw>::template load<AUX>(vr_, voff + uint32_t(i) * row_bytes, 0u);
        } else {
            kr[i] = IO::zero();
            vr[i] = IO::zero();
        }
    }
}

// Load this wave's n tokens of one array (the receptance) like chunk_load.
template <int DT, int VEC, int L, bool FULL, int AUX>
__device__ __forceinline__ void chunk_load_one(typename Io<DT, VEC>::Raw (&xr)[L], rsrc_t x_,
                                               uint32_t voff, uint32_t row_bytes, int n) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
#pragma unroll
    for (int i = 0; i < L; i++) {
        if (FULL || i < n)
            xr[i] = Buf<Raw>::template load<AUX>(x_, voff + uint32_t(i) * row_bytes, 0u);
        else
            xr[i] = IO::zero();
    }
}

// State of this wave's n tokens started from the empty history, by two
// passes: the largest decayed key x_i = k_i - (n-1-i) w, then the sums of
// e^{x_i - max} and e^{x_i - max} v_i.  This is the closed form of the
// recurrence over the tokens (the state's exponent is the running maximum),
// without a serial chain of maxima.
template <int DT, int VEC, int L, bool FULL, bool KEEP = true>
__device__ __forceinline__ void chunk_aggregate(const Lane<VEC>& s,
                                                const typename Io<DT, VEC>::Raw (&kr)[L],
                                                const typename Io<DT, VEC>::Raw (&vr)[L],
                                                int n, Part<VEC>& g) {
    using IO = Io<DT, VEC>;
    // short blocks keep the decayed keys of the first pass for the second
    // (unless the caller needs the registers: KEEP)
    constexpr bool kKeepX = KEEP && L <= 16;
    float xs[kKeepX ? L : 1][VEC];
    float mx[VEC];
#pragma unroll
    for (int q = 0; q < VEC; q++) mx[q] = kEmptyP;
#pragma unroll
    for (int i = 0; i < L; i++) {
        if (FULL || i < n) {
            const float ci = FULL ? float(i - (L - 1)) : float(i - (n - 1));
            float kf[VEC];
            IO::unpack(kr[i], kf);
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                const float x = __builtin_fmaf(ci, s.ch[q].w, kf[q]);
                if constexpr (kKeepX) xs[i][q] = x;
                mx[q] = __builtin_fmaxf(mx[q], x);
            }
        }
    }
    float mxl[VEC];
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        g.a[q] = 0.0f;
        g.b[q] = 0.0f;
        g.A[q] = mx[q];
        g.m[q] = 0.0f;
        mxl[q] = mx[q] * kLog2e;
    }
#pragma unroll
    for (int i = 0; i < L; i++) {
        if (FULL || i < n) {
            float kf[VEC], vf[VEC];
            if constexpr (!kKeepX) IO::unpack(kr[i], kf);
            IO::unpack(vr[i], vf);
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                float x;
                if constexpr (kKeepX) {
                    x = xs[i][q];
                } else {
                    const float ci = FULL ? float(i - (L - 1)) : float(i - (n - 1));
                    x = __builtin_fmaf(ci, s.ch[q].w, kf[q]);
                }
                // e^{x - max}; a rounding of max * log2e scales every term alike
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -mxl[q]));
                g.b[q] += e;
                g.a[q] = __builtin_fmaf(e, vf[q], g.a[q]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Frame weights: the output pass reuses the aggregate pass's exponentials.
//
// Inside a frame of F tokens the decay rides on the keys: in frame
// coordinates token i's key is x_i = k_i + (i + 1) w and the history (the
// state before the frame's first token, exponent H) decays no further
// (wkv_device.h, 4.).  The aggregate pass already forms e_i = e^{x_i - M}
// against the frame's largest key M.  Against G = max(H, M) the history
// takes alpha = e^{H-G} and the frame's tokens beta e_i with beta = e^{M-G}
// (one of the two is exactly 1), and token by token
//   y_i = (a + beta e_i c v_i) / (b + beta e_i c),  a += beta e_i v_i,
//   b += beta e_i,  starting from a = alpha a_H, b = alpha b_H,  c = e^{u-w}
// (the read-out of wkv_device.h 3. with the frame's weights fixed): no
// exponential, running maximum or select per token.  A history that keeps
// the maximum is not rescaled at all, as in frame_token.
//
// Fixing the weights for a whole frame needs them in range: the largest
// term of every prefix must stay a normal number, i.e. alpha (the history
// has b >= 1) or beta e_0 at least 2^-100 (with c >= 2^-20 the read-out's
// denominator stays above 2^-120).  A frame whose first token and history
// both sit more than 69 (natural-log units) below a later key of the frame
// fails that; if any lane of the wave does, the wave runs that frame token
// by token with the running maximum (frame_token), its keys read again.  On
// the bf16 workload (1 in 1000 keys at +-40) about 1 frame in 100 of a wave
// takes that path.
// ---------------------------------------------------------------------------

constexpr float kFrameTermMin = 7.88860905e-31f;  // 2^-100
constexpr float kFrameHistMax = 1.8446744e19f;    // 2^64: the history's weight against M_f

template <int VEC, int L>
struct FrameW {
    float e[L][VEC];                  // e^{x_i - M_f}
    float M[L / kFrameTokens][VEC];   // frame maxima M_f (natural-log units)
};

// Weights of a full block of L tokens (pass 1: frame keys and maxima; pass 2:
// e_i, with frame sums folded into g, the block's state from the empty
// history in anchor form).
template <int DT, int VEC, int L>
__device__ __forceinline__ void chunk_weights(const Lane<VEC>& s,
                                              const typename Io<DT, VEC>::Raw (&kr)[L],
                                              const typename Io<DT, VEC>::Raw (&vr)[L],
                                              FrameW<VEC, L>& fw, Part<VEC>& g) {
    using IO = Io<DT, VEC>;
    constexpr int F = kFrameTokens, NF = L / F;
    static_assert(L % F == 0 && F % 2 == 0, "whole frames of an even length");
#pragma unroll
    for (int f = 0; f < NF; f++) {
#pragma unroll
        for (int j = 0; j < F; j += 2) {
            const int i = f * F + j;
            float k0[VEC], k1[VEC];
            IO::unpack(kr[i], k0);
            IO::unpack(kr[i + 1], k1);
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                const float x0 = __builtin_fmaf(float(j + 1), s.ch[q].w, k0[q]);
                const float x1 = __builtin_fmaf(float(j + 2), s.ch[q].w, k1[q]);
                fw.e[i][q] = x0;
                fw.e[i + 1][q] = x1;
                fw.M[f][q] = j == 0 ? max_num(x0, x1) : max3_num(fw.M[f][q], x0, x1);
            }
        }
    }
#pragma unroll
    for (int f = 0; f < NF; f++) {
        float sa[VEC], sb[VEC];
#pragma unroll
        for (int q = 0; q < VEC; q++) { sa[q] = 0.0f; sb[q] = 0.0f; }
#pragma unroll
        for (int j = 0; j < F; j++) {
            const int i = f * F + j;
            float vf[VEC];
            IO::unpack(vr[i], vf);
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                // the difference first: exact 0 for the frame's largest key
                const float e = __builtin_amdgcn_exp2f((fw.e[i][q] - fw.M[f][q]) * kLog2e);
                fw.e[i][q] = e;
                sb[q] += e;
                sa[q] = __builtin_fmaf(e, vf[q], sa[q]);
            }
        }
        // frame f spans F tokens; its state in anchor form is (sa, sb, M_f, F)
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            if (f == 0) {
                g.a[q] = sa[q];
                g.b[q] = sb[q];
                g.A[q] = fw.M[0][q];
                g.m[q] = float(F);
            } else {
                combine(g.a[q], g.b[q], g.A[q], g.m[q], sa[q], sb[q], fw.M[f][q], float(F), float(F),
                        s.ch[q].w);
            }
        }
    }
}

// The outputs of a full block of L tokens from the state in s (anchor form),
// with the weights of chunk_weights; see above.  kr_, voff, row_bytes: where
// the block's keys are, for a frame that must run token by token.
template <int DT, int VEC, int L, bool GATED>
__device__ __forceinline__ void run_block_weights(Lane<VEC>& s, const FrameW<VEC, L>& fw,
                                                  const typename Io<DT, VEC>::Raw (&vr)[L],
                                                  const typename Io<DT, VEC>::Raw (&rr)[L],
                                                  rsrc_t kr_, rsrc_t yr_, uint32_t voff,
                                                  uint32_t row_bytes, bool active) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int F = kFrameTokens, NF = L / F;
#pragma unroll
    for (int f = 0; f < NF; f++) {
        float alpha[VEC], beta[VEC], H[VEC], hist[VEC];
        bool keep[VEC];
        bool ok = true, ok_anchor = true;
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            H[q] = __builtin_fmaf(-s.m[q], s.ch[q].w, s.A[q]);  // history exponent
            const float d = H[q] - fw.M[f][q];
            // the range checks look at the history's whole weight (factor * b),
            // so that a state whose b is far from 1 is safe too
            if constexpr (DT == kBF16) {
                // the history's factor against M_f (either side of 1)
                hist[q] = __builtin_amdgcn_exp2f(d * kLog2e);
                const float hb = hist[q] * s.b[q];
                ok_anchor = ok_anchor && hb <= kFrameHistMax &&
                            max_num(hb, fw.e[f * F][q]) >= kFrameTermMin;
            } else {
                const float e = exp_neg_abs(d);
                keep[q] = d >= 0.0f;
                alpha[q] = keep[q] ? 1.0f : e;
                beta[q] = keep[q] ? e : 1.0f;
                ok = ok && max_num(alpha[q] * s.b[q], beta[q] * fw.e[f * F][q]) >= kFrameTermMin;
            }
        }
        if (DT == kBF16 && __builtin_amdgcn_ballot_w64(!ok_anchor) == 0) {
            // bf16 storage: the frame's anchor is M_f whichever side keeps the
            // maximum, so the weights need no factor; the history is rescaled
            // by e^{H - M_f} <= 2^64 every frame (a rounding per frame, far
            // below one bf16 rounding of the output)
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                s.a[q] *= hist[q];
                s.b[q] *= hist[q];
            }
#pragma unroll
            for (int j = 0; j < F; j++) {
                const int i = f * F + j;
                float vf[VEC], yf[VEC], gd[VEC];
                IO::unpack(vr[i], vf);
                if constexpr (GATED) {
                    float rf[VEC];
                    IO::unpack(rr[i], rf);
#pragma unroll
                    for (int q = 0; q < VEC; q++) gd[q] = gate_den(rf[q]);
                }
#pragma unroll
                for (int q = 0; q < VEC; q++) {
                    const float e = fw.e[i][q];
                    const float ec = e * s.ch[q].c;
                    const float den = s.b[q] + ec;
                    yf[q] = __builtin_fmaf(ec, vf[q], s.a[q]) * fast_rcp(GATED ? den * gd[q] : den);
                    s.a[q] = __builtin_fmaf(e, vf[q], s.a[q]);
                    s.b[q] += e;
                }
                if (active) Buf<Raw>::template store<kStreamStore>(IO::pack(yf), yr_, voff, uint32_t(i) * row_bytes);
            }
#pragma unroll
            for (int q = 0; q < VEC; q++) { s.A[q] = fw.M[f][q]; s.m[q] = float(F); }
        } else if (DT != kBF16 && __builtin_amdgcn_ballot_w64(!ok) == 0) {
            float ct[VEC];
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                s.a[q] *= alpha[q];
                s.b[q] *= alpha[q];
                ct[q] = beta[q] * s.ch[q].c;
            }
#pragma unroll
            for (int j = 0; j < F; j++) {
                const int i = f * F + j;
                float vf[VEC], yf[VEC], gd[VEC];
                IO::unpack(vr[i], vf);
                if constexpr (GATED) {
                    float rf[VEC];
                    IO::unpack(rr[i], rf);
#pragma unroll
                    for (int q = 0; q < VEC; q++) gd[q] = gate_den(rf[q]);
                }
#pragma unroll
                for (int q = 0; q < VEC; q++) {
                    const float et = fw.e[i][q] * beta[q];
                    const float ec = fw.e[i][q] * ct[q];
                    const float den = s.b[q] + ec;
                    yf[q] = __builtin_fmaf(ec, vf[q], s.a[q]) * fast_rcp(GATED ? den * gd[q] : den);
                    s.a[q] = __builtin_fmaf(et, vf[q], s.a[q]);
                    s.b[q] += et;
                }
                if (active) Buf<Raw>::template store<kStreamStore>(IO::pack(yf), yr_, voff, uint32_t(i) * row_bytes);
            }
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                s.A[q] = keep[q] ? s.A[q] : fw.M[f][q];
                s.m[q] = keep[q] ? s.m[q] + float(F) : float(F);
            }
        } else {
            // token by token with the running maximum, the frame's keys read again
            float kas[VEC];
            bool all_keep[VEC];
#pragma unroll
            for (int q = 0; q < VEC; q++) { kas[q] = H[q]; all_keep[q] = true; }
#pragma unroll
            for (int j = 0; j < F; j++) {
                const int i = f * F + j;
                float kf[VEC], vf[VEC], yf[VEC], gd[VEC];
                IO::unpack(Buf<Raw>::template load<kDefaultLoad>(kr_, voff + uint32_t(i) * row_bytes, 0u), kf);
                IO::unpack(vr[i], vf);
                if constexpr (GATED) {
                    float rf[VEC];
                    IO::unpack(rr[i], rf);
#pragma unroll
                    for (int q = 0; q < VEC; q++) gd[q] = gate_den(rf[q]);
                }
#pragma unroll
                for (int q = 0; q < VEC; q++) {
                    bool kp;
                    yf[q] = frame_token<true, GATED>(s.a[q], s.b[q], kas[q], kf[q], vf[q], s.ch[q],
                                                     float(j + 1), kp, GATED ? gd[q] : 1.0f);
                    all_keep[q] = all_keep[q] && kp;
                }
                if (active) Buf<Raw>::template store<kStreamStore>(IO::pack(yf), yr_, voff, uint32_t(i) * row_bytes);
            }
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                s.A[q] = all_keep[q] ? s.A[q] : kas[q];
                s.m[q] = all_keep[q] ? s.m[q] + float(F) : float(F);
            }
        }
    }
}

// Materialise the weights and the aggregate here (an empty asm that takes
// and returns each of them in a register, ordered with the hand-off's
// volatile accesses).
template <int VEC, int L>
__device__ __forceinline__ void pin_weights(FrameW<VEC, L>& fw, Part<VEC>& g) {
#pragma unroll
    for (int i = 0; i < L; i++)
#pragma unroll
        for (int q = 0; q < VEC; q++) asm volatile("" : "+v"(fw.e[i][q]));
#pragma unroll
    for (int q = 0; q < VEC; q++)
        asm volatile("" : "+v"(g.a[q]), "+v"(g.b[q]), "+v"(g.A[q]), "+v"(g.m[q]));
}

// All channels of the wave may use the frame-weight output pass (fused
// read-out with c in [2^-20, 2^20]).
template <int VEC>
__device__ __forceinline__ bool wave_all_narrow(const Lane<VEC>& s) {
    bool f = true;
#pragma unroll
    for (int q = 0; q < VEC; q++) f = f && s.ch[q].narrow;
    return __builtin_amdgcn_ballot_w64(!f) == 0;
}

template <int DT, int VEC, bool GATED, int NW>
__global__ __launch_bounds__(NW * 64) void forward_chunked_kernel(ForwardProblem pr, ChunkArgs ca) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int L = kChunkTokens;
    constexpr int CG = 64 * VEC;
    constexpr int TILE = NW * L;
    // per-wave partial states, then their exclusive prefixes; [NW] = tile carry
    __shared__ float s_part[NW + 1][4][CG];
    __shared__ uint32_t s_ticket;

    const int wave = wave_id();
    const int lane = lane_id();
    if (threadIdx.x == 0) s_ticket = atomicAdd(ca.ticket, 1u);
    __syncthreads();
    const int64_t tile = __builtin_amdgcn_readfirstlane(s_ticket);
    const int64_t j = tile / ca.ngroups;
    const int64_t g = tile - j * ca.ngroups;
    const int64_t bb = g / ca.gpr;
    const int64_t c0 = (g - bb * ca.gpr) * CG;
    const int64_t c = c0 + int64_t(lane) * VEC;
    const bool active = c < pr.C;
    const int64_t T = pr.T;
    const int64_t t_begin = j * TILE + int64_t(wave) * L;
    const int n = T - t_begin >= L ? L : (T - t_begin > 0 ? int(T - t_begin) : 0);
    // lanes past the last channel take lane 0's channels: its data, parameters
    // and state, so they compute lane 0's values bit for bit and store lane
    // 0's bytes once more.  No store then needs a branch on the lane (one a
    // token cost about 1% of the bf16 workload's time)
    const int64_t cs = active ? c : c0;

    Lane<VEC> s;
    load_params(s, pr, cs, true);

    // k, v of this wave's tokens, kept in registers until y is written
    constexpr int64_t es = sizeof(Raw) / VEC;
    const uint32_t row_bytes = uint32_t(pr.C * es);
    const uint32_t voff = active ? uint32_t(lane) * uint32_t(sizeof(Raw)) : 0u;
    const int64_t base = ((bb * T + t_begin) * pr.C + c0) * es;
    Raw kr[L], vr[L], rr[GATED ? L : 1];
    {
        const rsrc_t kr_ = make_rsrc(static_cast<const char*>(pr.k) + base);
        const rsrc_t vr_ = make_rsrc(static_cast<const char*>(pr.v) + base);
        if (n == L)
            chunk_load<DT, VEC, L, true, kDefaultLoad>(kr, vr, kr_, vr_, voff, row_bytes, n);
        else
            chunk_load<DT, VEC, L, false, kDefaultLoad>(kr, vr, kr_, vr_, voff, row_bytes, n);
        if constexpr (GATED) {
            const rsrc_t rr_ = make_rsrc(static_cast<const char*>(pr.r) + base);
            if (n == L)
                chunk_load_one<DT, VEC, L, true, kDefaultLoad>(rr, rr_, voff, row_bytes, n);
            else
                chunk_load_one<DT, VEC, L, false, kDefaultLoad>(rr, rr_, voff, row_bytes, n);
        }
    }

    // phase 1: this wave's partial state from the empty history
    {
        Part<VEC> gw;
        if (n == L)
            chunk_aggregate<DT, VEC, L, true>(s, kr, vr, n, gw);
        else
            chunk_aggregate<DT, VEC, L, false>(s, kr, vr, n, gw);
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            s_part[wave][0][lane * VEC + q] = gw.a[q];
            s_part[wave][1][lane * VEC + q] = gw.b[q];
            s_part[wave][2][lane * VEC + q] = gw.A[q];
            s_part[wave][3][lane * VEC + q] = gw.m[q];
        }
    }
    __syncthreads();

    // wave 0: prefixes inside the tile, the tile's carry, publication
    if (wave == 0) {
        Part<VEC> pre;
        pre.set_empty();
        for (int w2 = 0; w2 < NW; w2++) {
            const int64_t tb = j * TILE + int64_t(w2) * L;
            const int n2 = T - tb >= L ? L : (T - tb > 0 ? int(T - tb) : 0);
            Part<VEC> gw;
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                gw.a[q] = s_part[w2][0][lane * VEC + q];
                gw.b[q] = s_part[w2][1][lane * VEC + q];
                gw.A[q] = s_part[w2][2][lane * VEC + q];
                gw.m[q] = s_part[w2][3][lane * VEC + q];
                s_part[w2][0][lane * VEC + q] = pre.a[q];
                s_part[w2][1][lane * VEC + q] = pre.b[q];
                s_part[w2][2][lane * VEC + q] = pre.A[q];
                s_part[w2][3][lane * VEC + q] = pre.m[q];
            }
            pre.absorb(gw, float(n2), s);
        }
        const int64_t tile_tokens = (T - j * TILE) < TILE ? (T - j * TILE) : TILE;
        const bool last_tile = j == ca.tiles_per_group - 1;
        Part<VEC> x;
        if (j == 0) {
            load_state(x.a, x.b, x.A, x.m, pr, bb * pr.C + cs, true);
        } else {
            if (!last_tile) publish<VEC>(ca, g, j, 0, pre, lane);
            look_back<VEC>(ca, g, j, TILE, s, x, lane);
        }
        if (!last_tile) {
            Part<VEC> inc = x;
            inc.absorb(pre, float(tile_tokens), s);
            publish<VEC>(ca, g, j, 1, inc, lane);
        }
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            s_part[NW][0][lane * VEC + q] = x.a[q];
            s_part[NW][1][lane * VEC + q] = x.b[q];
            s_part[NW][2][lane * VEC + q] = x.A[q];
            s_part[NW][3][lane * VEC + q] = x.m[q];
        }
    }
    __syncthreads();
    if (n == 0) return;

    // phase 3: carry-in of this wave, then the tokens again with outputs
    {
        Part<VEC> x;
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            x.a[q] = s_part[NW][0][lane * VEC + q];
            x.b[q] = s_part[NW][1][lane * VEC + q];
            x.A[q] = s_part[NW][2][lane * VEC + q];
            x.m[q] = s_part[NW][3][lane * VEC + q];
        }
        if (wave > 0) {
            Part<VEC> pw;
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                pw.a[q] = s_part[wave][0][lane * VEC + q];
                pw.b[q] = s_part[wave][1][lane * VEC + q];
                pw.A[q] = s_part[wave][2][lane * VEC + q];
                pw.m[q] = s_part[wave][3][lane * VEC + q];
            }
            x.absorb(pw, float(wave * L), s);
        }
#pragma unroll
        for (int q = 0; q < VEC; q++) { s.a[q] = x.a[q]; s.b[q] = x.b[q]; s.A[q] = x.A[q]; s.m[q] = x.m[q]; }
    }
    const rsrc_t yr_ = make_rsrc(static_cast<char*>(pr.y) + base);
    const bool fused = wave_all_fused(s);
    const Raw (&rg)[L] = gated_rr<GATED>(rr, kr);
    if (n == L) {
        if (fused)
            run_block<DT, VEC, L, true, true, GATED>(s, kr, vr, rg, yr_, voff, row_bytes, n, true);
        else
            run_block<DT, VEC, L, false, true, GATED>(s, kr, vr, rg, yr_, voff, row_bytes, n, true);
    } else {
        if (fused)
            run_block<DT, VEC, L, true, false, GATED>(s, kr, vr, rg, yr_, voff, row_bytes, n, true);
        else
            run_block<DT, VEC, L, false, false, GATED>(s, kr, vr, rg, yr_, voff, row_bytes, n, true);
    }
    if (t_begin + n == T && active && pr.a_out != nullptr) store_state(s, pr, bb * pr.C + c);
}

// ---------------------------------------------------------------------------
// chained path
//
// One workgroup of NWV waves owns a whole column group.  The group's tokens
// are cut into sub-chunks of kChainTokens tokens handed to the waves round-robin
// (sub-chunk c goes to wave c % NWV), kChainTokens tokens each.  For each of its sub-chunks a wave
// loads k, v into registers, folds them into a partial state from the empty
// history, then waits for the carry (the state before the sub-chunk) in LDS,
// passes on carry (+) partial to the next sub-chunk's wave, and re-runs its
// tokens from the carry to write y.  The carry chain costs one combine per
// sub-chunk; the loads and both passes of different waves overlap freely.
// No global memory besides k, v, y and the state is touched, and the result
// does not depend on timing.
// ---------------------------------------------------------------------------

// The carry of sub-chunk sc (the state before it) into s, and carry (+) gw
// (its n tokens) handed on to sub-chunk sc + 1 and returned in `after` (the
// state after the sub-chunk, anchored at the running maximum).  The hand-off is the
// workgroup's critical path (every wave waits on it in turn), so the wave
// runs it at raised issue priority over the others' passes.
template <int VEC>
__device__ __forceinline__ void chain_handoff(Lane<VEC>& s, const Part<VEC>& gw, int n, int64_t sc,
                                              int64_t nsub, float (&s_carry)[4][64 * VEC],
                                              int* s_seq, int lane, Part<VEC>& after) {
    __builtin_amdgcn_s_setprio(3);
    while (__hip_atomic_load(s_seq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != int(sc))
        __builtin_amdgcn_s_sleep(1);
    Part<VEC> x;
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        x.a[q] = s_carry[0][lane * VEC + q];
        x.b[q] = s_carry[1][lane * VEC + q];
        x.A[q] = s_carry[2][lane * VEC + q];
        x.m[q] = s_carry[3][lane * VEC + q];
    }
    after = x;
    after.absorb(gw, float(n), s);
    if (sc + 1 < nsub) {
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            s_carry[0][lane * VEC + q] = after.a[q];
            s_carry[1][lane * VEC + q] = after.b[q];
            s_carry[2][lane * VEC + q] = after.A[q];
            s_carry[3][lane * VEC + q] = after.m[q];
        }
        if (lane == 0) __hip_atomic_store(s_seq, int(sc + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int q = 0; q < VEC; q++) { s.a[q] = x.a[q]; s.b[q] = x.b[q]; s.A[q] = x.A[q]; s.m[q] = x.m[q]; }
}

// The carry of sub-chunk sc (the state before it, in s) to pr.states
// [B][nsub][r, q][C] (to_saved): the backward's checkpoints.
template <int VEC>
__device__ __forceinline__ void save_carry(const Lane<VEC>& s, const ForwardProblem& pr, int64_t bb,
                                           int64_t sc, int64_t nsub, int64_t c, bool active) {
    if (!active) return;
    float r[VEC], q[VEC];
#pragma unroll
    for (int i = 0; i < VEC; i++)
        to_saved(s.a[i], s.b[i], __builtin_fmaf(-s.m[i], s.ch[i].w, s.A[i]), r[i], q[i]);
    // non-temporal stores (read once, by the backward): the saving forward
    // 172 -> 161-167 us on the bf16 workload, against plain stores
    const rsrc_t so = make_rsrc(pr.states + (bb * nsub + sc) * 2 * pr.C);
    const uint32_t field = uint32_t(pr.C) * uint32_t(sizeof(float));
    if constexpr (VEC == 2) {
        // one 8-byte store per field (c is even and the rows 8-byte aligned)
        Buf<float2>::template store<kNonTemporalStore>(make_float2(r[0], r[1]), so, uint32_t(c) * 4u, 0u);
        Buf<float2>::template store<kNonTemporalStore>(make_float2(q[0], q[1]), so, uint32_t(c) * 4u, field);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; i++) {
            Buf<float>::template store<kNonTemporalStore>(r[i], so, uint32_t(c + i) * 4u, 0u);
            Buf<float>::template store<kNonTemporalStore>(q[i], so, uint32_t(c + i) * 4u, field);
        }
    }
}

// SAVE: each sub-chunk's carry also goes to pr.states (save_carry).
template <int DT, int VEC, int NWV, bool GATED, bool SAVE>
__global__ __launch_bounds__(NWV * 64) void forward_chained_kernel(ForwardProblem pr, int64_t gpr,
                                                                   int64_t nsub) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int L = kChainTokens;
    constexpr int CG = 64 * VEC;
    __shared__ float s_carry[4][CG];  // a, b, A, m of the state before sub-chunk s_seq
    __shared__ int s_seq;

    const int wave = wave_id();
    const int lane = lane_id();
    const int64_t g = blockIdx.x;
    const int64_t bb = g / gpr;
    const int64_t c0 = (g - bb * gpr) * CG;
    const int64_t c = c0 + int64_t(lane) * VEC;
    const bool active = c < pr.C;
    const int64_t T = pr.T;
    // lanes past the last channel mirror lane 0, as on the chunked path
    const int64_t cs = active ? c : c0;

    Lane<VEC> s;
    load_params(s, pr, cs, true);
    if (wave == 0) {
        float a[VEC], b[VEC], A[VEC], m[VEC];
        load_state(a, b, A, m, pr, bb * pr.C + cs, true);
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            s_carry[0][lane * VEC + q] = a[q];
            s_carry[1][lane * VEC + q] = b[q];
            s_carry[2][lane * VEC + q] = A[q];
            s_carry[3][lane * VEC + q] = m[q];
        }
        if (lane == 0) s_seq = 0;
    }
    __syncthreads();

    constexpr int64_t es = sizeof(Raw) / VEC;
    const uint32_t row_bytes = uint32_t(pr.C * es);
    const uint32_t voff = active ? uint32_t(lane) * uint32_t(sizeof(Raw)) : 0u;
    const int64_t gbase = (bb * T * pr.C + c0) * es;
    const bool fused = wave_all_fused(s);
    const bool narrow = wave_all_narrow(s);

    for (int64_t sc = wave; sc < nsub; sc += NWV) {
        const int64_t t0 = sc * L;
        const int n = T - t0 >= L ? L : int(T - t0);
        const int64_t base = gbase + t0 * int64_t(row_bytes);
        Part<VEC> after;   // the state after this sub-chunk (exported after the last)
        const rsrc_t kr_ = make_rsrc(static_cast<const char*>(pr.k) + base);
        const rsrc_t vr_ = make_rsrc(static_cast<const char*>(pr.v) + base);
        const rsrc_t yr_ = make_rsrc(static_cast<char*>(pr.y) + base);
        // the receptance is needed only after the carry: its loads are issued
        // after the aggregate, to overlap the wait for the carry
        if (narrow && n == L) {
            // frame weights: the keys are done with after the aggregate pass
            Raw kr[L], vr[L], rr[GATED ? L : 1];
            FrameW<VEC, L> fw;
            Part<VEC> gw;
            chunk_load<DT, VEC, L, true, kStreamLoad>(kr, vr, kr_, vr_, voff, row_bytes, n);
            chunk_weights<DT, VEC, L>(s, kr, vr, fw, gw);
            if constexpr (GATED)
                chunk_load_one<DT, VEC, L, true, kStreamLoad>(
                    rr, make_rsrc(static_cast<const char*>(pr.r) + base), voff, row_bytes, n);
            // the weights and the aggregate are finished before the wait for the
            // carry: left to itself the compiler sinks them below it, onto the
            // chain of hand-offs that every wave of the workgroup waits on
            pin_weights(fw, gw);
            chain_handoff<VEC>(s, gw, n, sc, nsub, s_carry, &s_seq, lane, after);
            if constexpr (SAVE) save_carry(s, pr, bb, sc, nsub, c, active);
            run_block_weights<DT, VEC, L, GATED>(s, fw, vr, gated_rr<GATED>(rr, kr), kr_, yr_, voff,
                                                 row_bytes, true);
        } else {
            Raw kr[L], vr[L], rr[GATED ? L : 1];
            Part<VEC> gw;
            if (n == L) {
                chunk_load<DT, VEC, L, true, kStreamLoad>(kr, vr, kr_, vr_, voff, row_bytes, n);
                chunk_aggregate<DT, VEC, L, true, !GATED>(s, kr, vr, n, gw);
                if constexpr (GATED)
                    chunk_load_one<DT, VEC, L, true, kStreamLoad>(
                        rr, make_rsrc(static_cast<const char*>(pr.r) + base), voff, row_bytes, n);
            } else {
                chunk_load<DT, VEC, L, false, kStreamLoad>(kr, vr, kr_, vr_, voff, row_bytes, n);
                chunk_aggregate<DT, VEC, L, false, !GATED>(s, kr, vr, n, gw);
                if constexpr (GATED)
                    chunk_load_one<DT, VEC, L, false, kStreamLoad>(
                        rr, make_rsrc(static_cast<const char*>(pr.r) + base), voff, row_bytes, n);
            }
            chain_handoff<VEC>(s, gw, n, sc, nsub, s_carry, &s_seq, lane, after);
            if constexpr (SAVE) save_carry(s, pr, bb, sc, nsub, c, active);
            const Raw (&rg)[L] = gated_rr<GATED>(rr, kr);
            if (n == L) {
                if (fused)
                    run_block<DT, VEC, L, true, true, GATED>(s, kr, vr, rg, yr_, voff, row_bytes, n, true);
                else
                    run_block<DT, VEC, L, false, true, GATED>(s, kr, vr, rg, yr_, voff, row_bytes, n, true);
            } else {
                if (fused)
                    run_block<DT, VEC, L, true, false, GATED>(s, kr, vr, rg, yr_, voff, row_bytes, n, true);
                else
                    run_block<DT, VEC, L, false, false, GATED>(s, kr, vr, rg, yr_, voff, row_bytes, n, true);
            }
        }
        if (sc == nsub - 1 && active && pr.a_out != nullptr) {
#pragma unroll
            for (int q = 0; q < VEC; q++) { s.a[q] = after.a[q]; s.b[q] = after.b[q]; s.A[q] = after.A[q]; s.m[q] = after.m[q]; }
            store_state(s, pr, bb * pr.C + c);
        }
    }
}

// Clears the tile dispenser, the error flag and the n tile flags.
__global__ void reset_chunk_counters(uint32_t* ticket, uint64_t* flags, int64_t n) {
    const int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i0 == 0) {
        ticket[0] = 0u;  // tile dispenser
        ticket[1] = 0u;  // look-back error flag
    }
    for (int64_t i = i0; i < n; i += int64_t(gridDim.x) * blockDim.x) flags[i] = kEmpty;
}

__global__ void state_passthrough_kernel(int64_t n, const float* a_in, const float* b_in,
                                         const float* p_in, float* a_out, float* b_out,
                                         float* p_out) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if (a_in != nullptr) {
        const float a = a_in[i], b = b_in[i], p = p_in[i];
        a_out[i] = a;
        b_out[i] = b;
        p_out[i] = export_p(clamp_empty(p));  // empty inputs come back as -inf
    } else {
        a_out[i] = 0.0f;
        b_out[i] = 0.0f;
        p_out[i] = -__builtin_inff();
    }
}

}  // namespace

int pick_forward_vec(int64_t C, int dtype, bool aligned) {
    if (dtype == kBF16 && C % 2 == 0 && aligned) return 2;
    return 1;
}

ChunkPlan plan_chunked(int64_t B, int64_t T, int64_t C, int vec, int waves) {
    ChunkPlan pl;
    pl.vec = vec;
    const int64_t cg = 64 * pl.vec;
    const int64_t gpr = (C + cg - 1) / cg;
    pl.ngroups = B * gpr;
    if (waves == 0) {
        // tiles of 8 waves; of 16 when the 8-wave tiles would outnumber the
        // CUs and the 16-wave ones would not (B=8 T=1024 C=768 fp32: 384 tiles
        // of 8 waves in 21.2 us, 192 of 16 in 19.2 us; at B=1 T=65536 C=4096,
        // 16-wave tiles ran 610 against 577 us, and 4-wave tiles or 16-token
        // waves were slower everywhere)
        const int64_t cus = device_cu_count();
        const int64_t t8 = pl.ngroups * ((T + kChunkTokens * kChunkWaves - 1) / (kChunkTokens * kChunkWaves));
        const int64_t t16 = pl.ngroups * ((T + kChunkTokens * kChunkWavesWide - 1) / (kChunkTokens * kChunkWavesWide));
        waves = (t8 > cus && t16 <= cus) ? kChunkWavesWide : kChunkWaves;
    }
    pl.waves = waves;
    pl.tile_tokens = kChunkTokens * waves;
    pl.tiles_per_group = (T + pl.tile_tokens - 1) / pl.tile_tokens;
    const size_t ntiles = size_t(pl.ngroups) * size_t(pl.tiles_per_group);
    const size_t flags = (ntiles * sizeof(uint64_t) + 255) & ~size_t(255);
    const size_t desc = ntiles * 2 * 4 * size_t(cg) * sizeof(float);
    pl.workspace_bytes = ntiles == 0 ? 0 : 256 + flags + desc;
    return pl;
}

size_t forward_workspace_bytes(int64_t B, int64_t T, int64_t C, int dtype, int path) {
    if (path != 2 || T == 0) return 0;
    // the size query does not see the pointers: cover both lane widths
    // and 8-wave tiles: the chosen width may be 16 waves, whose fewer tiles
    // need less
    const size_t w1 = plan_chunked(B, T, C, 1, kChunkWaves).workspace_bytes;
    const size_t w2 = plan_chunked(B, T, C, pick_forward_vec(C, dtype, true), kChunkWaves).workspace_bytes;
    return w1 > w2 ? w1 : w2;
}

int choose_forward_path(const ForwardProblem& pr, int device_cus) {
    const int64_t cg = 64 * pr.vec;
    const int64_t ngroups = pr.B * ((pr.C + cg - 1) / cg);
    if (pr.T <= kChunkTokens) return 1;                       // a single block
    if (ngroups >= int64_t(device_cus) * 16) return 1;        // 4 waves per SIMD without splitting T
    if (4 * ngroups >= 3 * int64_t(device_cus)) return 3;     // a workgroup per column group fills the chip
    return 2;                                                 // split T across workgroups
}

int chained_waves(int64_t ngroups, int device_cus) {
    // enough waves per workgroup for 16 per CU, a power of two in [2, 16]
    int nw = 16;
    while (nw > 2 && int64_t(nw) * ngroups > int64_t(device_cus) * 16) nw /= 2;
    return nw;
}

namespace {
template <bool GATED, bool SAVE>
void launch_chained_t(const ForwardProblem& pr, int nw, dim3 grid, int64_t gpr, int64_t nsub,
                      hipStream_t stream) {
    const dim3 block(nw * 64);
#define WKV_LAUNCH_CHAINED(DT, V, NW)                                                             \
    hipLaunchKernelGGL((forward_chained_kernel<DT, V, NW, GATED, SAVE>), grid, block, 0, stream, pr, \
                       gpr, nsub)
#define WKV_CHAINED_NW(DT, V)                                   \
    switch (nw) {                                              \
        case 16: WKV_LAUNCH_CHAINED(DT, V, 16); break;         \
        case 8: WKV_LAUNCH_CHAINED(DT, V, 8); break;           \
        case 4: WKV_LAUNCH_CHAINED(DT, V, 4); break;           \
        default: WKV_LAUNCH_CHAINED(DT, V, 2); break;          \
    }
    if (pr.dtype == kBF16 && pr.vec == 2) {
        WKV_CHAINED_NW(kBF16, 2)
    } else if (pr.dtype == kBF16) {
        WKV_CHAINED_NW(kBF16, 1)
    } else {
        WKV_CHAINED_NW(kF32, 1)
    }
#undef WKV_CHAINED_NW
#undef WKV_LAUNCH_CHAINED
}
}  // namespace

hipError_t launch_forward_chained(const ForwardProblem& pr, hipStream_t stream) {
    const int64_t cg = 64 * pr.vec;
    const int64_t gpr = (pr.C + cg - 1) / cg;
    const int64_t ngroups = pr.B * gpr;
    const int64_t nsub = (pr.T + kChainTokens - 1) / kChainTokens;
    const int nw = chained_waves(ngroups, device_cu_count());
    const dim3 grid(static_cast<unsigned>(ngroups));
    // saved states are the backward's checkpoints: one per 16 tokens
    if (pr.states != nullptr && (pr.r != nullptr || kChainTokens != WKV_SAVED_STATE_TOKENS))
        return hipErrorInvalidValue;
    if (pr.r != nullptr)
        launch_chained_t<true, false>(pr, nw, grid, gpr, nsub, stream);
    else if (pr.states != nullptr)
        launch_chained_t<false, true>(pr, nw, grid, gpr, nsub, stream);
    else
        launch_chained_t<false, false>(pr, nw, grid, gpr, nsub, stream);
    return hipGetLastError();
}

namespace {
template <bool GATED>
void launch_serial_t(const ForwardProblem& pr, dim3 grid, int64_t ngroups, int64_t gpr,
                     hipStream_t stream) {
    const dim3 block(kSerialWaves * 64);
    if (pr.dtype == kBF16 && pr.vec == 2)
        hipLaunchKernelGGL((forward_serial_kernel<kBF16, 2, GATED>), grid, block, 0, stream, pr, ngroups, gpr);
    else if (pr.dtype == kBF16)
        hipLaunchKernelGGL((forward_serial_kernel<kBF16, 1, GATED>), grid, block, 0, stream, pr, ngroups, gpr);
    else
        hipLaunchKernelGGL((forward_serial_kernel<kF32, 1, GATED>), grid, block, 0, stream, pr, ngroups, gpr);
}
}  // namespace

hipError_t launch_forward_serial(const ForwardProblem& pr, hipStream_t stream) {
    const int64_t cg = 64 * pr.vec;
    const int64_t gpr = (pr.C + cg - 1) / cg;
    const int64_t ngroups = pr.B * gpr;
    const int64_t blocks = (ngroups + kSerialWaves - 1) / kSerialWaves;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (pr.r != nullptr)
        launch_serial_t<true>(pr, grid, ngroups, gpr, stream);
    else
        launch_serial_t<false>(pr, grid, ngroups, gpr, stream);
    return hipGetLastError();
}

namespace {
template <bool GATED, int NW>
void launch_chunked_nw(const ForwardProblem& pr, const ChunkArgs& ca, int vec, dim3 grid,
                       hipStream_t stream) {
    const dim3 block(NW * 64);
    if (pr.dtype == kBF16 && vec == 2)
        hipLaunchKernelGGL((forward_chunked_kernel<kBF16, 2, GATED, NW>), grid, block, 0, stream, pr, ca);
    else if (pr.dtype == kBF16)
        hipLaunchKernelGGL((forward_chunked_kernel<kBF16, 1, GATED, NW>), grid, block, 0, stream, pr, ca);
    else
        hipLaunchKernelGGL((forward_chunked_kernel<kF32, 1, GATED, NW>), grid, block, 0, stream, pr, ca);
}
template <bool GATED>
void launch_chunked_t(const ForwardProblem& pr, const ChunkArgs& ca, int vec, int waves, dim3 grid,
                      hipStream_t stream) {
    if (waves == kChunkWavesWide)
        launch_chunked_nw<GATED, kChunkWavesWide>(pr, ca, vec, grid, stream);
    else
        launch_chunked_nw<GATED, kChunkWaves>(pr, ca, vec, grid, stream);
}
}  // namespace

hipError_t launch_forward_chunked(const ForwardProblem& pr, void* workspace, hipStream_t stream) {
    const ChunkPlan pl = plan_chunked(pr.B, pr.T, pr.C, pr.vec);
    ChunkArgs ca;
    ca.ngroups = pl.ngroups;
    ca.gpr = pl.ngroups / pr.B;
    ca.tiles_per_group = pl.tiles_per_group;
    char* ws = static_cast<char*>(workspace);
    ca.ticket = reinterpret_cast<uint32_t*>(ws);
    ca.error = ca.ticket + 1;
    const size_t ntiles = size_t(pl.ngroups) * size_t(pl.tiles_per_group);
    const size_t flags = (ntiles * sizeof(uint64_t) + 255) & ~size_t(255);
    ca.flags = reinterpret_cast<uint64_t*>(ws + 256);
    ca.desc = reinterpret_cast<float*>(ws + 256 + flags);
    const int64_t reset_blocks = std::min<int64_t>((int64_t(ntiles) + 255) / 256, 1024);
    hipLaunchKernelGGL(reset_chunk_counters, dim3(static_cast<unsigned>(reset_blocks)), dim3(256), 0,
                       stream, ca.ticket, ca.flags, int64_t(ntiles));
    const dim3 grid(static_cast<unsigned>(ntiles));
    if (pr.r != nullptr)
        launch_chunked_t<true>(pr, ca, pl.vec, pl.waves, grid, stream);
    else
        launch_chunked_t<false>(pr, ca, pl.vec, pl.waves, grid, stream);
    return hipGetLastError();
}

hipError_t read_chunk_wait_failures(uint64_t* count) {
    unsigned int n = 0;
    const hipError_t e = hipMemcpyFromSymbol(&n, HIP_SYMBOL(g_chunk_wait_failures), sizeof(n), 0,
                                             hipMemcpyDeviceToHost);
    *count = n;
    return e;
}

hipError_t launch_state_passthrough(const ForwardProblem& pr, hipStream_t stream) {
    const int64_t n = pr.B * pr.C;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(state_passthrough_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, n,
                       pr.a_in, pr.b_in, pr.p_in, pr.a_out, pr.b_out, pr.p_out);
    return hipGetLastError();
}

}  // namespace wkv
