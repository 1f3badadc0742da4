// wkv_backward: gradients of L = sum(gy * wkv) with respect to k, v, w and u
// for wkv_forward from the empty history.  Each wkv_t is a weighted mean of
// values with weights e^{-(t-1-i)w + k_i} (i < t) and e^{u + k_t} ([tm-math]
// = aicassindra.com tm_rwkv_math, "The WKV operator"), so with D_t the sum of
// the weights:
//
//   gv_i = gy_i e^{u+k_i} / D_i + e^{k_i} P_i
//   gk_i = gy_i e^{u+k_i} (v_i - y_i) / D_i + e^{k_i} (v_i P_i - Q_i)
//   gu   = sum_t gy_t e^{u+k_t} (v_t - y_t) / D_t
//   gw   = -sum_t gy_t (A'_t - y_t B'_t) / D_t
//
// where P_i = sum_{t>i} e^{-(t-1-i)w} gy_t / D_t and Q_i the same with
// gy_t y_t (a scan backwards in time: P_{i-1} = gy_i / D_i + e^{-w} P_i),
// A_t, B_t the history sums of the forward recurrence and A'_t, B'_t the
// same weighted by age t-1-i (a scan forwards: A'_{t+1} = e^{-w} (A'_t +
// A_t)).  gw and gu are summed over B and T.
//
// Execution (one workgroup of NWV waves per column group = 64 lanes x VEC
// channels of one batch row; the tokens cut into sub-chunks of kBwdTokens,
// handed to the waves round-robin as on the forward's chained path):
//
//   phase F  forward in time.  Each wave loads k, v of its sub-chunk and
//            sums them into a partial state (a, b, a', b') from the empty
//            history (max of the exponents, then the sum); the carry (the state before the sub-chunk) arrives
//            through LDS, carry (+) partial goes on to the next sub-chunk, and
//            the carry is stored to the workspace as that sub-chunk's
//            checkpoint.
//   phase R  backward in time, sub-chunks from the last.  Each wave loads
//            k, v, gy and its checkpoint, re-runs the forward recurrence over
//            the sub-chunk (outputs y_t, 1/D_t, the gu and gw terms) and
//            sums the sub-chunk's (P, Q) contribution into a partial; the
//            (P, Q) carry from the later sub-chunk arrives through LDS,
//            carry (+) partial goes on to the earlier one, and the tokens are
//            walked backwards from the carry to write gk, gv.
//
// Stabilisation: every scale is an exponent in anchor form, anchor - count w,
// and every weight an exponential of a non-positive difference formed
// anchor-relative: (anchor - key) is exact when the two are close, and the
// count w term is added by one fma at the difference's own magnitude, so no
// rounding at the keys' magnitude accumulates through the rescalings.  The
// (P, Q) scan is held against e^{-q_t} with the factor 1/delta_t = e^{q_t} /
// D_t folded into its terms; q_t is an exponent the read-out already has (the
// larger of the history's and u + k_t, or the folded state's plus w when the
// read-out reuses the fold's weights), so delta_t lies in [min(1, e^{u-w}),
// tokens] and e^{k_i} times the scan's scale stays <= 1.
//
// gw, gu are reduced per column over the waves in LDS (fixed order), stored
// per (b, c), and summed over the batch by a last kernel in batch order: the
// result does not depend on timing.
#include "wkv_device.h"
#include "wkv_internal.h"

#include <type_traits>

namespace wkv {
namespace {

constexpr int kBwdTokens = 16;  // tokens per sub-chunk
constexpr int kCkptFields = 6;  // a, b, a', b', anchor, count

__device__ __forceinline__ int bwd_wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int bwd_lane_id() { return threadIdx.x & 63; }

// Forward state in anchor form: exponent p = A - m w; a, b the history sums
// and ap, bp the age-weighted ones, all scaled by e^{-p}.
struct FState {
    float a, b, ap, bp, A, m;
    __device__ __forceinline__ void set_empty() {
        a = b = ap = bp = 0.0f;
        A = kEmptyP;
        m = 0.0f;
    }
};

// X <- X (+) G, G the state of the n tokens after X from the empty history.
// Over n tokens X's terms gain n in age: a' -> e^{-n w} (a' + n a).
__device__ __forceinline__ void combine_forward(FState& x, const FState& g, float n, float w) {
    const float d = __builtin_fmaf(-(x.m + n - g.m), w, x.A - g.A);  // X's exponent - G's
    const float e = exp_neg_abs(d);
    const bool keep = d >= 0.0f;
    const float ax = keep ? 1.0f : e;
    const float ag = keep ? e : 1.0f;
    const float apx = __builtin_fmaf(n, x.a, x.ap);
    const float bpx = __builtin_fmaf(n, x.b, x.bp);
    x.a = __builtin_fmaf(ax, x.a, ag * g.a);
    x.b = __builtin_fmaf(ax, x.b, ag * g.b);
    x.ap = __builtin_fmaf(ax, apx, ag * g.ap);
    x.bp = __builtin_fmaf(ax, bpx, ag * g.bp);
    x.A = keep ? x.A : g.A;
    x.m = keep ? x.m + n : g.m;
}

// Reverse accumulator (P, Q) in anchor form: exponent Pi - n w.
struct RState {
    float P, Q, Pi, n;
    __device__ __forceinline__ void set_empty() {
        P = Q = 0.0f;
        Pi = kEmptyP;
        n = 0.0f;
    }
};

// X <- X (+) G for the reverse scan: X holds the tokens after a span of n
// tokens (its exponent gains -n w at the span's start), G the span's own.
__device__ __forceinline__ void combine_reverse(RState& x, const RState& g, float n, float w) {
    const float d = __builtin_fmaf(-(x.n + n - g.n), w, x.Pi - g.Pi);
    const float e = exp_neg_abs(d);
    const bool keep = d >= 0.0f;
    const float ax = keep ? 1.0f : e;
    const float ag = keep ? e : 1.0f;
    x.P = __builtin_fmaf(ax, x.P, ag * g.P);
    x.Q = __builtin_fmaf(ax, x.Q, ag * g.Q);
    x.Pi = keep ? x.Pi : g.Pi;
    x.n = keep ? x.n + n : g.n;
}

// Per-token values the backward walk needs, per channel.
struct TokenOut {
    float y;   // the output wkv_t
    float q;   // the read-out's larger exponent
    float gr;  // gy_t / delta_t  (gy_t / D_t = gr e^{-q})
    float ed;  // gy_t e^{u+k_t} / D_t
};

// The forward read-out of one token from state s, its gw, gu terms, then the
// fold-in.  FUSED (|u - w| <= 44, c = e^{u-w} in range): the read-out reuses
// the fold's weights, as the forward kernels do -- relative to the folded
// exponent p' = max(p - w, k), the history weighs al = e^{p-w-p'}, the new
// token be = e^{k-p'}, and D = e^{p'+w} (al b + be c) -- so one exponential
// serves both; the (P, Q) exponent is then q = p' + w.  Otherwise the
// read-out takes its own exponential against q = max(p, u + k).
template <bool FUSED>
__device__ __forceinline__ TokenOut forward_detail(FState& s, float k, float v, float g, float w,
                                                   float u, float c, float& gw, float& gu) {
    TokenOut o;
    const float ak = s.A - k;
    const float e = __builtin_fmaf(-(s.m + 1.0f), w, ak);  // (p - w) - k
    const float x = exp_neg_abs(e);
    const bool reset = e < 0.0f;                             // the new key is the maximum
    const float al = reset ? x : 1.0f;
    const float be = reset ? 1.0f : x;
    float rh, bo;  // read-out weights of history and bonus, relative to e^{q}
    if constexpr (FUSED) {
        rh = al;
        bo = be * c;
        // the folded exponent plus w: k + w on a reset, else A - m w (the
        // same roundings either way: fma(1, w, k) is k + w)
        o.q = __builtin_fmaf(reset ? 1.0f : -s.m, w, reset ? k : s.A);
    } else {
        const float d = __builtin_fmaf(-s.m, w, ak - u);  // p - (u + k)
        const float xr = exp_neg_abs(d);
        const bool keep = d >= 0.0f;
        rh = keep ? 1.0f : xr;
        bo = keep ? xr : 1.0f;
        // u + k is rounded as in d's reference point
        o.q = keep ? __builtin_fmaf(-s.m, w, s.A) : u + k;
    }
    const float del = __builtin_fmaf(rh, s.b, bo);
    const float rd = fast_rcp(del);
    o.y = __builtin_fmaf(rh, s.a, bo * v) * rd;
    o.gr = g * rd;
    o.ed = o.gr * bo;
    gu = __builtin_fmaf(o.ed, v - o.y, gu);
    gw = __builtin_fmaf(-(o.gr * rh), __builtin_fmaf(-o.y, s.bp, s.ap), gw);
    // fold-in: the history decays by e^{-w}, the age-weighted sums gain the
    // history, the new key enters with weight e^{k}
    s.ap = al * (s.ap + s.a);
    s.bp = al * (s.bp + s.b);
    s.a = __builtin_fmaf(al, s.a, be * v);
    s.b = __builtin_fmaf(al, s.b, be);
    s.A = reset ? k : s.A;
    s.m = reset ? 0.0f : s.m + 1.0f;
    return o;
}

// The first n tokens of a sub-chunk through forward_detail.
template <typename IO, int L, int VEC, bool FUSED, typename Raw>
__device__ __forceinline__ void forward_run(FState (&s)[VEC], const Raw (&kr)[L], const Raw (&vr)[L],
                                            const Raw (&gyr)[L], const float (&w)[VEC],
                                            const float (&u)[VEC], const float (&c)[VEC], int n,
                                            TokenOut (&to)[L][VEC], float (&gw)[VEC],
                                            float (&gu)[VEC]) {
#pragma unroll
    for (int i = 0; i < L; i++) {
        if (i < n) {
            float kf[VEC], vf[VEC], gf[VEC];
            IO::unpack(kr[i], kf);
            IO::unpack(vr[i], vf);
            IO::unpack(gyr[i], gf);
#pragma unroll
            for (int q = 0; q < VEC; q++)
                to[i][q] = forward_detail<FUSED>(s[q], kf[q], vf[q], gf[q], w[q], u[q], c[q], gw[q], gu[q]);
        }
    }
}

// One token of the backward walk: gk, gv from the running (P, Q) of the
// later tokens, then fold this token's term in (skipped for a sub-chunk's
// first token, whose successor is the next sub-chunk's carry).
__device__ __forceinline__ void reverse_detail(RState& r, const TokenOut& o, float k, float v, float w,
                                               bool fold, float& gk, float& gv) {
    const float eh = __builtin_amdgcn_exp2f(__builtin_fmaf(-r.n, w, k + r.Pi) * kLog2e);
    gv = __builtin_fmaf(eh, r.P, o.ed);
    gk = __builtin_fmaf(eh, __builtin_fmaf(v, r.P, -r.Q), o.ed * (v - o.y));
    if (fold) {
        const float e = __builtin_fmaf(-(r.n + 1.0f), w, r.Pi + o.q);  // (pi - w) - (-q)
        const float x = exp_neg_abs(e);
        const bool reset = e < 0.0f;
        const float al = reset ? x : 1.0f;
        const float be = reset ? 1.0f : x;
        const float t = be * o.gr;
        r.P = __builtin_fmaf(al, r.P, t);
        r.Q = __builtin_fmaf(al, r.Q, t * o.y);
        r.Pi = reset ? -o.q : r.Pi;
        r.n = reset ? 0.0f : r.n + 1.0f;
    }
}

template <int DT, int VEC, int NWV>
__global__ __launch_bounds__(NWV * 64) void backward_chained_kernel(BackwardProblem pr, int64_t gpr,
                                                                    int64_t nsub) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int L = kBwdTokens;
    constexpr int CG = 64 * VEC;
    __shared__ float s_fc[kCkptFields][CG];  // forward carry before sub-chunk s_fseq
    __shared__ float s_rc[4][CG];            // reverse carry after sub-chunk nsub-1-s_rseq
    __shared__ float s_red[2][NWV][CG];      // per-wave gw, gu
    __shared__ int s_fseq, s_rseq;

    const int wave = bwd_wave_id();
    const int lane = bwd_lane_id();
    const int64_t grp = blockIdx.x;
    const int64_t bb = grp / gpr;
    const int64_t c0 = (grp - bb * gpr) * CG;
    const int64_t c = c0 + int64_t(lane) * VEC;
    const bool active = c < pr.C;
    const int64_t T = pr.T, C = pr.C;

    float w[VEC], u[VEC], cb[VEC];
    bool fus = true;
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        w[q] = active ? pr.w[c + q] : 1.0f;
        u[q] = active ? pr.u[c + q] : 0.0f;
        const float wmu = w[q] - u[q];
        fus = fus && __builtin_fabsf(wmu) <= kFusedMaxAbsUW;
        cb[q] = __builtin_amdgcn_exp2f(-wmu * kLog2e);  // e^{u-w}
    }
    const bool fused = __builtin_amdgcn_ballot_w64(!fus) == 0;
    if (wave == 0) {
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            FState e;
            e.set_empty();
            s_fc[0][lane * VEC + q] = e.a;
            s_fc[1][lane * VEC + q] = e.b;
            s_fc[2][lane * VEC + q] = e.ap;
            s_fc[3][lane * VEC + q] = e.bp;
            s_fc[4][lane * VEC + q] = e.A;
            s_fc[5][lane * VEC + q] = e.m;
            RState r;
            r.set_empty();
            s_rc[0][lane * VEC + q] = r.P;
            s_rc[1][lane * VEC + q] = r.Q;
            s_rc[2][lane * VEC + q] = r.Pi;
            s_rc[3][lane * VEC + q] = r.n;
        }
        if (lane == 0) {
            s_fseq = 0;
            s_rseq = 0;
        }
    }
    __syncthreads();

    constexpr int64_t es = sizeof(Raw) / VEC;
    const uint32_t row_bytes = uint32_t(C * es);
    const uint32_t voff = active ? uint32_t(lane) * uint32_t(sizeof(Raw)) : 0u;
    uint32_t toff[L];
#pragma unroll
    for (int i = 0; i < L; i++) toff[i] = voff + uint32_t(i) * row_bytes;
    const int64_t gbase = (bb * T * C + c0) * es;
    // checkpoints: [B][nsub][field][C] fp32
    float* ckpt = pr.ckpt + bb * nsub * kCkptFields * C + c;

    // ---------------- phase F: forward carries and checkpoints ----------------
    for (int64_t sc = wave; sc < nsub; sc += NWV) {
        const int64_t t0 = sc * L;
        const int n = T - t0 >= L ? L : int(T - t0);
        const int64_t base = gbase + t0 * int64_t(row_bytes);
        const rsrc_t kr_ = make_rsrc(static_cast<const char*>(pr.k) + base);
        const rsrc_t vr_ = make_rsrc(static_cast<const char*>(pr.v) + base);
        Raw kr[L], vr[L];
#pragma unroll
        for (int i = 0; i < L; i++) {
            if (i < n) {
                kr[i] = Buf<Raw>::template load<kStreamLoad>(kr_, toff[i], 0);
                vr[i] = Buf<Raw>::template load<kStreamLoad>(vr_, toff[i], 0);
            }
        }
        // the sub-chunk from the empty history, max then sum: token i has
        // exponent x_i = k_i - (n-1-i) w at the sub-chunk's end; the partial's
        // anchor is the largest, each weight e^{x_i - max}
        FState g[VEC];
        {
            float xs[L][VEC], mx[VEC];
#pragma unroll
            for (int q = 0; q < VEC; q++) mx[q] = kEmptyP;
#pragma unroll
            for (int i = 0; i < L; i++) {
                if (i < n) {
                    float kf[VEC];
                    IO::unpack(kr[i], kf);
#pragma unroll
                    for (int q = 0; q < VEC; q++) {
                        xs[i][q] = __builtin_fmaf(-float(n - 1 - i), w[q], kf[q]);
                        mx[q] = max_num(mx[q], xs[i][q]);
                    }
                }
            }
            // e^{x_i - max}; a rounding of max * log2e scales every term alike
            float mxl[VEC];
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                g[q].set_empty();
                g[q].A = mx[q];
                mxl[q] = mx[q] * kLog2e;
            }
#pragma unroll
            for (int i = 0; i < L; i++) {
                if (i < n) {
                    float vf[VEC];
                    IO::unpack(vr[i], vf);
                    const float age = float(n - 1 - i);
#pragma unroll
                    for (int q = 0; q < VEC; q++) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[i][q], kLog2e, -mxl[q]));
                        const float ev = e * vf[q];
                        g[q].a += ev;
                        g[q].b += e;
                        g[q].ap = __builtin_fmaf(age, ev, g[q].ap);
                        g[q].bp = __builtin_fmaf(age, e, g[q].bp);
                    }
                }
            }
        }
        while (__hip_atomic_load(&s_fseq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != int(sc))
            __builtin_amdgcn_s_sleep(1);
        FState x[VEC];
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            x[q].a = s_fc[0][lane * VEC + q];
            x[q].b = s_fc[1][lane * VEC + q];
            x[q].ap = s_fc[2][lane * VEC + q];
            x[q].bp = s_fc[3][lane * VEC + q];
            x[q].A = s_fc[4][lane * VEC + q];
            x[q].m = s_fc[5][lane * VEC + q];
        }
        if (sc + 1 < nsub) {
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                FState nx = x[q];
                combine_forward(nx, g[q], float(n), w[q]);
                s_fc[0][lane * VEC + q] = nx.a;
                s_fc[1][lane * VEC + q] = nx.b;
                s_fc[2][lane * VEC + q] = nx.ap;
                s_fc[3][lane * VEC + q] = nx.bp;
                s_fc[4][lane * VEC + q] = nx.A;
                s_fc[5][lane * VEC + q] = nx.m;
            }
            if (lane == 0)
                __hip_atomic_store(&s_fseq, int(sc + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (active) {
            float* ck = ckpt + sc * kCkptFields * C;
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                ck[0 * C + q] = x[q].a;
                ck[1 * C + q] = x[q].b;
                ck[2 * C + q] = x[q].ap;
                ck[3 * C + q] = x[q].bp;
                ck[4 * C + q] = x[q].A;
                ck[5 * C + q] = x[q].m;
            }
        }
    }
    // every checkpoint is written (and visible to the workgroup) past here
    __syncthreads();

    // ---------------- phase R: the backward walk ----------------
    float gw[VEC], gu[VEC];
#pragma unroll
    for (int q = 0; q < VEC; q++) gw[q] = gu[q] = 0.0f;
    // the read-out form is uniform over the workgroup (its waves share the
    // channels): one copy of the loop per form keeps their registers apart
    auto reverse_phase = [&](auto fused_tag) {
        for (int64_t j = wave; j < nsub; j += NWV) {
            const int64_t sc = nsub - 1 - j;
            const int64_t t0 = sc * L;
            const int n = T - t0 >= L ? L : int(T - t0);
            const int64_t base = gbase + t0 * int64_t(row_bytes);
            const rsrc_t kr_ = make_rsrc(static_cast<const char*>(pr.k) + base);
            const rsrc_t vr_ = make_rsrc(static_cast<const char*>(pr.v) + base);
            const rsrc_t gr_ = make_rsrc(static_cast<const char*>(pr.gy) + base);
            Raw kr[L], vr[L], gyr[L];
    #pragma unroll
            for (int i = 0; i < L; i++) {
                if (i < n) {
                    kr[i] = Buf<Raw>::template load<kStreamLoad>(kr_, toff[i], 0);
                    vr[i] = Buf<Raw>::template load<kStreamLoad>(vr_, toff[i], 0);
                    gyr[i] = Buf<Raw>::template load<kStreamLoad>(gr_, toff[i], 0);
                }
            }
            FState s[VEC];
            {
                const float* ck = ckpt + sc * kCkptFields * C;
    #pragma unroll
                for (int q = 0; q < VEC; q++) {
                    s[q].a = ck[0 * C + q];
                    s[q].b = ck[1 * C + q];
                    s[q].ap = ck[2 * C + q];
                    s[q].bp = ck[3 * C + q];
                    s[q].A = ck[4 * C + q];
                    s[q].m = ck[5 * C + q];
                }
            }
            TokenOut to[L][VEC];
            forward_run<IO, L, VEC, decltype(fused_tag)::value>(s, kr, vr, gyr, w, u, cb, n, to, gw, gu);
            // the sub-chunk's (P, Q) partial, max then sum: token i's term has
            // exponent -q_i - i w at the sub-chunk's start
            RState rg[VEC];
            {
                float mx[VEC];
    #pragma unroll
                for (int q = 0; q < VEC; q++) mx[q] = kEmptyP;
    #pragma unroll
                for (int i = 0; i < L; i++)
                    if (i < n)
    #pragma unroll
                        for (int q = 0; q < VEC; q++)
                            mx[q] = max_num(mx[q], __builtin_fmaf(-float(i), w[q], -to[i][q].q));
                float mxl[VEC];
    #pragma unroll
                for (int q = 0; q < VEC; q++) {
                    rg[q].set_empty();
                    rg[q].Pi = mx[q];
                    mxl[q] = mx[q] * kLog2e;
                }
    #pragma unroll
                for (int i = 0; i < L; i++) {
                    if (i < n) {
    #pragma unroll
                        for (int q = 0; q < VEC; q++) {
                            const float xi = __builtin_fmaf(-float(i), w[q], -to[i][q].q);
                            const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(xi, kLog2e, -mxl[q])) * to[i][q].gr;
                            rg[q].P += t;
                            rg[q].Q = __builtin_fmaf(t, to[i][q].y, rg[q].Q);
                        }
                    }
                }
            }
            while (__hip_atomic_load(&s_rseq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != int(j))
                __builtin_amdgcn_s_sleep(1);
            RState r[VEC];
    #pragma unroll
            for (int q = 0; q < VEC; q++) {
                r[q].P = s_rc[0][lane * VEC + q];
                r[q].Q = s_rc[1][lane * VEC + q];
                r[q].Pi = s_rc[2][lane * VEC + q];
                r[q].n = s_rc[3][lane * VEC + q];
            }
            if (sc > 0) {
    #pragma unroll
                for (int q = 0; q < VEC; q++) {
                    RState nr = r[q];
                    combine_reverse(nr, rg[q], float(n), w[q]);
                    s_rc[0][lane * VEC + q] = nr.P;
                    s_rc[1][lane * VEC + q] = nr.Q;
                    s_rc[2][lane * VEC + q] = nr.Pi;
                    s_rc[3][lane * VEC + q] = nr.n;
                }
                if (lane == 0)
                    __hip_atomic_store(&s_rseq, int(j + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            const rsrc_t gkr_ = make_rsrc(static_cast<char*>(pr.gk) + base);
            const rsrc_t gvr_ = make_rsrc(static_cast<char*>(pr.gv) + base);
    #pragma unroll
            for (int i = L - 1; i >= 0; i--) {
                if (i < n) {
                    float kf[VEC], vf[VEC], gkf[VEC], gvf[VEC];
                    IO::unpack(kr[i], kf);
                    IO::unpack(vr[i], vf);
    #pragma unroll
                    for (int q = 0; q < VEC; q++)
                        reverse_detail(r[q], to[i][q], kf[q], vf[q], w[q], i > 0, gkf[q], gvf[q]);
                    if (active) {
                        Buf<Raw>::store(IO::pack(gkf), gkr_, toff[i], 0);
                        Buf<Raw>::store(IO::pack(gvf), gvr_, toff[i], 0);
                    }
                }
            }
        }
    };
    if (fused)
        reverse_phase(std::integral_constant<bool, true>{});
    else
        reverse_phase(std::integral_constant<bool, false>{});

    // ---------------- gw, gu of this (b, column group) ----------------
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        s_red[0][wave][lane * VEC + q] = gw[q];
        s_red[1][wave][lane * VEC + q] = gu[q];
    }
    __syncthreads();
    if (wave == 0 && active) {
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            float sw = 0.0f, su = 0.0f;
            for (int v2 = 0; v2 < NWV; v2++) {
                sw += s_red[0][v2][lane * VEC + q];
                su += s_red[1][v2][lane * VEC + q];
            }
            pr.part_w[bb * C + c + q] = sw;
            pr.part_u[bb * C + c + q] = su;
        }
    }
}

// gw[c] = sum_b part_w[b][c], gu likewise, in batch order.
__global__ void backward_reduce(BackwardProblem pr) {
    const int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (c >= pr.C) return;
    float sw = 0.0f, su = 0.0f;
    for (int64_t bb = 0; bb < pr.B; bb++) {
        sw += pr.part_w[bb * pr.C + c];
        su += pr.part_u[bb * pr.C + c];
    }
    pr.gw[c] = sw;
    pr.gu[c] = su;
}

__global__ void zero_pair(float* x, float* y, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) {
        x[i] = 0.0f;
        y[i] = 0.0f;
    }
}

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int backward_vec(int64_t C, int dtype, bool aligned) {
    return (dtype == kBF16 && C % 2 == 0 && aligned) ? 2 : 1;
}

size_t backward_workspace_bytes(int64_t B, int64_t T, int64_t C) {
    const size_t nsub = size_t((T + kBwdTokens - 1) / kBwdTokens);
    const size_t cols = size_t(B) * size_t(C);
    return up256(cols * nsub * kCkptFields * 4) + 2 * up256(cols * 4);
}

hipError_t launch_backward(BackwardProblem pr, void* workspace, hipStream_t stream) {
    if (pr.T == 0) {
        hipLaunchKernelGGL(zero_pair, dim3(unsigned((pr.C + 255) / 256)), dim3(256), 0, stream, pr.gw,
                           pr.gu, pr.C);
        return hipGetLastError();
    }
    const int64_t cols = pr.B * pr.C;
    const int64_t nsub = (pr.T + kBwdTokens - 1) / kBwdTokens;
    char* ws = static_cast<char*>(workspace);
    pr.ckpt = reinterpret_cast<float*>(ws);
    const size_t ck = up256(size_t(cols) * size_t(nsub) * kCkptFields * 4);
    pr.part_w = reinterpret_cast<float*>(ws + ck);
    pr.part_u = reinterpret_cast<float*>(ws + ck + up256(size_t(cols) * 4));
    const int64_t cg = 64 * pr.vec;
    const int64_t gpr = (pr.C + cg - 1) / cg;
    const dim3 grid(unsigned(pr.B * gpr));
    constexpr int NW = 8;
    const dim3 block(NW * 64);
    if (pr.dtype == kBF16 && pr.vec == 2)
        hipLaunchKernelGGL((backward_chained_kernel<kBF16, 2, NW>), grid, block, 0, stream, pr, gpr, nsub);
    else if (pr.dtype == kBF16)
        hipLaunchKernelGGL((backward_chained_kernel<kBF16, 1, NW>), grid, block, 0, stream, pr, gpr, nsub);
    else
        hipLaunchKernelGGL((backward_chained_kernel<kF32, 1, NW>), grid, block, 0, stream, pr, gpr, nsub);
    hipLaunchKernelGGL(backward_reduce, dim3(unsigned((pr.C + 255) / 256)), dim3(256), 0, stream, pr);
    return hipGetLastError();
}

}  // namespace wkv
