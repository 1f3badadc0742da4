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
//   phase F  forward in time (skipped when a saving forward has stored the
//            states).  Each wave loads k, v of its sub-chunk and sums them
//            into a partial state (a, b) from the empty history (max of the
//            exponents, then the sum); the carry (the state before the
//            sub-chunk) arrives through LDS, carry (+) partial goes on to the
//            next sub-chunk, and the carry is stored to the workspace as that
//            sub-chunk's checkpoint (two numbers per channel).
//   phase R  backward in time, sub-chunks from the last.  Each wave loads
//            k, v, gy and its checkpoint, re-runs the forward recurrence over
//            the sub-chunk (y_t and gy_t / D_t) and sums the sub-chunk's
//            (P, Q, R, U) contribution into a partial; the carry from the
//            later sub-chunk arrives through LDS, carry (+) partial goes on to
//            the earlier one, and the tokens are walked backwards from the
//            carry to write gk, gv and sum the gw, gu terms.  Full
//            sub-chunks of channels with c = e^{u-w} in [2^-20, 2^20] run in
//            frames of 8 tokens with one exponential per token (below);
//            sub-chunks whose values leave the frames' range, and ragged
//            ones, run token by token.
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
static_assert(kBwdTokens == WKV_SAVED_STATE_TOKENS, "saved states are the checkpoints");
constexpr int kCkptFields = 2;  // r, q (to_saved)

__device__ __forceinline__ int bwd_wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int bwd_lane_id() { return threadIdx.x & 63; }

// Forward state in anchor form: exponent p = A - m w; a, b the history sums
// scaled by e^{-p}.  The same form as the forward kernels' carry; the
// checkpoints between the phases (and the states a saving forward hands
// over) keep it in two numbers per channel (to_saved / from_saved).
struct FState {
    float a, b, A, m;
    __device__ __forceinline__ void set_empty() {
        a = b = 0.0f;
        A = kEmptyP;
        m = 0.0f;
    }
};

// X <- X (+) G, G the state of the n tokens after X from the empty history.
__device__ __forceinline__ void combine_forward(FState& x, const FState& g, float n, float w) {
    const float d = __builtin_fmaf(-(x.m + n - g.m), w, x.A - g.A);  // X's exponent - G's
    const float e = exp_neg_abs(d);
    const bool keep = d >= 0.0f;
    const float ax = keep ? 1.0f : e;
    const float ag = keep ? e : 1.0f;
    x.a = __builtin_fmaf(ax, x.a, ag * g.a);
    x.b = __builtin_fmaf(ax, x.b, ag * g.b);
    x.A = keep ? x.A : g.A;
    x.m = keep ? x.m + n : g.m;
}

// Reverse accumulators in anchor form, exponent Pi - n w: P, Q the sums of
// gy_t / D_t and gy_t y_t / D_t over the later tokens, each decayed by its
// distance, and R, U the same weighted by that distance.
struct RState {
    float P, Q, R, U, Pi, n;
    __device__ __forceinline__ void set_empty() {
        P = Q = R = U = 0.0f;
        Pi = kEmptyP;
        n = 0.0f;
    }
};

// X <- X (+) G for the reverse scan: X holds the tokens after a span of n
// tokens (its exponent gains -n w at the span's start, and its terms n in
// distance: R -> e^{-n w} (R + n P)), G the span's own.
__device__ __forceinline__ void combine_reverse(RState& x, const RState& g, float n, float w) {
    const float d = __builtin_fmaf(-(x.n + n - g.n), w, x.Pi - g.Pi);
    const float e = exp_neg_abs(d);
    const bool keep = d >= 0.0f;
    const float ax = keep ? 1.0f : e;
    const float ag = keep ? e : 1.0f;
    const float Rx = __builtin_fmaf(n, x.P, x.R);
    const float Ux = __builtin_fmaf(n, x.Q, x.U);
    x.P = __builtin_fmaf(ax, x.P, ag * g.P);
    x.Q = __builtin_fmaf(ax, x.Q, ag * g.Q);
    x.R = __builtin_fmaf(ax, Rx, ag * g.R);
    x.U = __builtin_fmaf(ax, Ux, ag * g.U);
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

// The forward read-out of one token from state s, its gu term, then the
// fold-in.  FUSED (|u - w| <= 44, c = e^{u-w} in range): the read-out reuses
// the fold's weights, as the forward kernels do -- relative to the folded
// exponent p' = max(p - w, k), the history weighs al = e^{p-w-p'}, the new
// token be = e^{k-p'}, and D = e^{p'+w} (al b + be c) -- so one exponential
// serves both; the (P, Q) exponent is then q = p' + w.  Otherwise the
// read-out takes its own exponential against q = max(p, u + k).
template <bool FUSED>
__device__ __forceinline__ TokenOut forward_detail(FState& s, float k, float v, float g, float w,
                                                   float u, float c, float& gu) {
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
    // fold-in: the history decays by e^{-w}, the new key enters with weight
    // e^{k}
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
                                            TokenOut (&to)[L][VEC], float (&gu)[VEC]) {
#pragma unroll
    for (int i = 0; i < L; i++) {
        if (i < n) {
            float kf[VEC], vf[VEC], gf[VEC];
            IO::unpack(kr[i], kf);
            IO::unpack(vr[i], vf);
            IO::unpack(gyr[i], gf);
#pragma unroll
            for (int q = 0; q < VEC; q++)
                to[i][q] = forward_detail<FUSED>(s[q], kf[q], vf[q], gf[q], w[q], u[q], c[q], gu[q]);
        }
    }
}

// One token of the backward walk: gk, gv and the token's gw term,
// -e^{k} (v R - U), from the running sums of the later tokens, then fold this
// token's term in (skipped for a sub-chunk's first token, whose successor is
// the next sub-chunk's carry).  Moving one token back, every later term gains
// one in distance: R -> e^{-w} (R + P), with P before this token's term.
__device__ __forceinline__ void reverse_detail(RState& r, const TokenOut& o, float k, float v, float w,
                                               bool fold, float& gk, float& gv, float& gw) {
    const float eh = __builtin_amdgcn_exp2f(__builtin_fmaf(-r.n, w, k + r.Pi) * kLog2e);
    gv = __builtin_fmaf(eh, r.P, o.ed);
    gk = __builtin_fmaf(eh, __builtin_fmaf(v, r.P, -r.Q), o.ed * (v - o.y));
    gw = __builtin_fmaf(-eh, __builtin_fmaf(v, r.R, -r.U), gw);
    if (fold) {
        const float e = __builtin_fmaf(-(r.n + 1.0f), w, r.Pi + o.q);  // (pi - w) - (-q)
        const float x = exp_neg_abs(e);
        const bool reset = e < 0.0f;
        const float al = reset ? x : 1.0f;
        const float be = reset ? 1.0f : x;
        const float t = be * o.gr;
        r.R = al * (r.R + r.P);
        r.U = al * (r.U + r.Q);
        r.P = __builtin_fmaf(al, r.P, t);
        r.Q = __builtin_fmaf(al, r.Q, t * o.y);
        r.Pi = reset ? -o.q : r.Pi;
        r.n = reset ? 0.0f : r.n + 1.0f;
    }
}

// ---------------------------------------------------------------------------
// Frame weights in the backward walk (full sub-chunks of channels with the
// fused read-out and c = e^{u-w} in [2^-20, 2^20]).
//
// Inside a frame of kBwdFrame tokens the decay rides on the keys: in frame
// coordinates token i's key is x_i = k_i + (i + 1) w, the history (exponent
// H) decays no further, and against one anchor G = max(H, M) per frame (M the
// frame's largest key) every weight is e_i = e^{x_i - G} <= 1 and the
// history's factor e^{H - G} <= 1 ([tm-math] "Why it collapses into a
// recurrence").  Token by token, with den_i = b + e_i c:
//   D_t = e^{G - i w} den_i,   y = (a + e_i c v) / den_i,
//   gy / D_t = e^{-(G - i w)} gr,  gr = gy / den_i,
//   gy e^{u+k} / D_t = gr e_i c,   a += e_i v, b += e_i
// and for the walk backwards, with S, SQ the sums of gr, gr y over the later
// tokens of the frame plus the later frames' carried in, and S2, SQ2 the same
// weighted by the distance (no decay: it rides on the weights):
//   e^{k_t} P_t = e_t S,  e^{k_t} Q_t = e_t SQ,  e^{k_t} R_t = e_t S2, ...
// A frame's sums go on to the frame before it with the factor
// e^{G_prev - F w - G} <= 1 (the next frame's anchor is at least the previous
// one's, decayed over the frame), and to the sub-chunk before through the
// carry's anchor form at exponent -G of the first frame.  No exponential per
// token but the weight itself.
//
// Fixed weights need the values in range for every lane that holds a channel
// (lanes past the last channel compute on stand-in data and are not asked;
// their results are never stored): the first prefix of
// each frame (the history, whose b is at least 1 against its own exponent,
// or the first token) at least 2^-100 of the anchor (so every den is a
// normal number), every token's weight normal, and every gy / den at most
// 2^100 (so the walk's sums cannot overflow).  A sub-chunk that fails any runs token by token
// (forward_detail, reverse_detail); so does a walk whose carried-in sums
// overflow.
// ---------------------------------------------------------------------------

constexpr int kBwdFrame = 8;
constexpr int kBwdFrames = kBwdTokens / kBwdFrame;
constexpr float kBwdTermMin = 7.88860905e-31f;   // 2^-100
constexpr float kBwdWeightMin = 1.17549435e-38f; // 2^-126, fp32's smallest normal
constexpr float kBwdGrMax = 1.26765060e30f;      // 2^100

// Per token and channel of a frame-weight sub-chunk the walk needs the
// weight against the frame's anchor (kept in registers) and the output y
// and gy / den.  Those two sit in registers (FrameYG) or, for two channels a
// lane, in a per-wave LDS stash (16 tokens x 64 lanes x 16 bytes): the walk
// runs after the hand-off, and holding them across it would take the whole
// register file.
template <int VEC>
struct FrameYG {
    float y[kBwdTokens][VEC], gr[kBwdTokens][VEC];
};
template <int VEC, bool STASH>
struct FrameStore;
template <int VEC>
struct FrameStore<VEC, false> {
    FrameYG<VEC> r;
    __device__ __forceinline__ void put(int i, const float (&y)[VEC], const float (&gr)[VEC]) {
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            r.y[i][q] = y[q];
            r.gr[i][q] = gr[q];
        }
    }
    __device__ __forceinline__ void get(int i, float (&y)[VEC], float (&gr)[VEC]) const {
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            y[q] = r.y[i][q];
            gr[q] = r.gr[i][q];
        }
    }
};
template <>
struct FrameStore<2, true> {
    float4* p;  // this wave's stash, [token][lane]
    int lane;
    __device__ __forceinline__ void put(int i, const float (&y)[2], const float (&gr)[2]) {
        p[i * 64 + lane] = make_float4(y[0], gr[0], y[1], gr[1]);
    }
    __device__ __forceinline__ void get(int i, float (&y)[2], float (&gr)[2]) const {
        const float4 t = p[i * 64 + lane];
        y[0] = t.x;
        gr[0] = t.y;
        y[1] = t.z;
        gr[1] = t.w;
    }
};

// The forward re-run of a full sub-chunk in frames from the checkpoint s0:
// the sub-chunk's own partial of the reverse sums.  Returns false for the
// whole wave when some lane's values leave the range.
template <typename IO, int L, int VEC, typename Raw, typename Store>
__device__ __forceinline__ bool frames_rerun(const FState (&s0)[VEC], const Raw (&kr)[L],
                                             const Raw (&vr)[L], const Raw (&gyr)[L],
                                             const float (&w)[VEC], const float (&c)[VEC],
                                             float (&te)[L][VEC], Store& st, float (&G)[kBwdFrames][VEC],
                                             float (&rho)[kBwdFrames][VEC], RState (&rg)[VEC],
                                             bool active) {
    constexpr int F = kBwdFrame, NF = kBwdFrames;
    static_assert(L == F * NF, "whole frames");
    // frame keys x and frame maxima M; the frame anchors G, each the larger of
    // M and the history's exponent H at the frame's start (H of the first
    // frame from the checkpoint, of the next G - F w); then the weights
    // e^{x - G}, all at most 1
    float M[NF][VEC], H0[VEC];
#pragma unroll
    for (int f = 0; f < NF; f++) {
#pragma unroll
        for (int j = 0; j < F; j++) {
            const int i = f * F + j;
            float kf[VEC];
            IO::unpack(kr[i], kf);
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                const float x = __builtin_fmaf(float(j + 1), w[q], kf[q]);
                te[i][q] = x;
                M[f][q] = j == 0 ? x : max_num(M[f][q], x);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        H0[q] = __builtin_fmaf(-s0[q].m, w[q], s0[q].A);
        float h = H0[q];
#pragma unroll
        for (int f = 0; f < NF; f++) {
            G[f][q] = max_num(h, M[f][q]);
            h = __builtin_fmaf(-float(F), w[q], G[f][q]);
        }
    }
#pragma unroll
    for (int f = 0; f < NF; f++) {
#pragma unroll
        for (int j = 0; j < F; j++) {
            const int i = f * F + j;
#pragma unroll
            for (int q = 0; q < VEC; q++)
                te[i][q] = __builtin_amdgcn_exp2f((te[i][q] - G[f][q]) * kLog2e);
        }
    }
    // per frame: the sums of gr and gr y over its tokens, and the same
    // weighted by the token's place in the sub-chunk; they enter the partial
    // (P, Q, R, U, at the first frame's anchor) with pi, the product of the
    // factors rho of the frames before
    float a[VEC], b[VEC], pi[VEC], sg[VEC], sq[VEC], sgi[VEC], sqi[VEC];
    float P[VEC], Q[VEC], R[VEC], U[VEC];
    float grmax = 0.0f, emin = 1.0f;
    bool ok = true;
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        a[q] = s0[q].a;
        b[q] = s0[q].b;
        pi[q] = 1.0f;
        P[q] = Q[q] = R[q] = U[q] = 0.0f;
    }
#pragma unroll
    for (int f = 0; f < NF; f++) {
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            // the history's sums move to the frame's anchor: e^{H - G} <= 1.
            // For a later frame H = G_{f-1} - F w, and the same factor
            // carries the frame's reverse sums into the frame before (rho)
            const float x = f == 0 ? H0[q] - G[0][q]
                                   : __builtin_fmaf(-float(F), w[q], G[f - 1][q] - G[f][q]);
            const float alpha = __builtin_amdgcn_exp2f(x * kLog2e);
            ok &= max_num(alpha * b[q], te[f * F][q]) >= kBwdTermMin;
            a[q] *= alpha;
            b[q] *= alpha;
            sg[q] = 0.0f;
            sq[q] = 0.0f;
            sgi[q] = 0.0f;
            sqi[q] = 0.0f;
            if (f > 0) {
                rho[f - 1][q] = alpha;
                pi[q] *= alpha;
            }
        }
        if (__builtin_amdgcn_ballot_w64(!ok & active) != 0) return false;
#pragma unroll
        for (int j = 0; j < F; j++) {
            const int i = f * F + j;
            float vf[VEC], gf[VEC];
            IO::unpack(vr[i], vf);
            IO::unpack(gyr[i], gf);
            float yt[VEC], grt[VEC];
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                const float et = te[i][q];
                const float ec = et * c[q];
                const float rd = fast_rcp(b[q] + ec);
                const float y = __builtin_fmaf(ec, vf[q], a[q]) * rd;
                const float gr = gf[q] * rd;
                const float gry = gr * y;
                a[q] = __builtin_fmaf(et, vf[q], a[q]);
                b[q] += et;
                sg[q] += gr;
                sq[q] += gry;
                sgi[q] = __builtin_fmaf(float(i), gr, sgi[q]);
                sqi[q] = __builtin_fmaf(float(i), gry, sqi[q]);
                grmax = max_num(grmax, __builtin_fabsf(gr));
                emin = min_num(emin, et);
                yt[q] = y;
                grt[q] = gr;
            }
            st.put(i, yt, grt);
            // token after token: left free, the scheduler runs the cheap
            // prefix chains ahead over the frame and holds every token's
            // values at once
#pragma unroll
            for (int q = 0; q < VEC; q++)
                asm volatile("" : "+v"(a[q]), "+v"(b[q]), "+v"(sg[q]), "+v"(sq[q]), "+v"(sgi[q]),
                             "+v"(sqi[q]));
        }
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            P[q] = __builtin_fmaf(pi[q], sg[q], P[q]);
            Q[q] = __builtin_fmaf(pi[q], sq[q], Q[q]);
            R[q] = __builtin_fmaf(pi[q], sgi[q], R[q]);
            U[q] = __builtin_fmaf(pi[q], sqi[q], U[q]);
        }
    }
    // gy / den beyond 2^100 (or not finite), or a weight below fp32's
    // smallest normal, for some lane: token by token.  A token's gk, gv are
    // its weight times the walk's sums, and a flushed or subnormal weight
    // would lose their relative precision however large the sums are
    if (__builtin_amdgcn_ballot_w64((!(grmax <= kBwdGrMax) | !(emin >= kBwdWeightMin)) & active) != 0)
        return false;
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        // the partial at the sub-chunk's start: exponent -G of the first frame
        rg[q].P = P[q];
        rg[q].Q = Q[q];
        rg[q].R = R[q];
        rg[q].U = U[q];
        rg[q].Pi = -G[0][q];
        rg[q].n = 0.0f;
    }
    return true;
}

// The walk of a frame-weight sub-chunk from the carry r after it (exponent
// r.Pi - r.n w at the sub-chunk's last token): gk, gv of every token, and the
// sub-chunk's gw and gu terms in gw, gu (for the caller to add).  Returns
// false, writing nothing, when the carried-in sums overflow fp32 for some lane
// of the wave.
template <typename IO, int L, int VEC, typename Raw, typename Store>
__device__ __forceinline__ bool frames_walk(const RState (&r)[VEC], const float (&te)[L][VEC],
                                            const Store& st,
                                            const float (&G)[kBwdFrames][VEC],
                                            const float (&rho)[kBwdFrames][VEC], const Raw (&vr)[L],
                                            const float (&w)[VEC], const float (&c)[VEC],
                                            rsrc_t gkr_, rsrc_t gvr_, uint32_t voff, uint32_t row_bytes,
                                            bool active, float (&gw)[VEC], float (&gu)[VEC]) {
    constexpr int F = kBwdFrame, NF = kBwdFrames;
    // S, SQ: the sums of gr, gr y over the later tokens; S2, SQ2 the same
    // weighted by the distance past the current token (both in frame
    // coordinates)
    float S[VEC], SQ[VEC], S2[VEC], SQ2[VEC];
    bool ok = true;
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        // e^{G_last - F w + exponent of the carry}, applied in two halves:
        // the factor alone may overflow where its product with the carry
        // (a tiny P after a small gy) does not
        const float x = __builtin_fmaf(-(r[q].n + float(F)), w[q], G[NF - 1][q] + r[q].Pi);
        const float h = __builtin_amdgcn_exp2f(x * (0.5f * kLog2e));
        S[q] = (h * r[q].P) * h;
        SQ[q] = (h * r[q].Q) * h;
        S2[q] = (h * r[q].R) * h;
        SQ2[q] = (h * r[q].U) * h;
        ok &= __builtin_isfinite(S[q]) & __builtin_isfinite(SQ[q]) & __builtin_isfinite(S2[q]) &
              __builtin_isfinite(SQ2[q]);
        gw[q] = 0.0f;
        gu[q] = 0.0f;
    }
    if (__builtin_amdgcn_ballot_w64(!ok & active) != 0) return false;
#pragma unroll
    for (int f = NF - 1; f >= 0; f--) {
        if (f < NF - 1) {
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                S[q] *= rho[f][q];
                SQ[q] *= rho[f][q];
                S2[q] *= rho[f][q];
                SQ2[q] *= rho[f][q];
            }
        }
        // the frame's y, gy / den, read in the order they are used, all
        // before the first is needed: read token by token, each read's LDS
        // latency stood in the walk's way
        float yt[F][VEC], grt[F][VEC];
#pragma unroll
        for (int j = F - 1; j >= 0; j--) st.get(f * F + j, yt[j], grt[j]);
#pragma unroll
        for (int j = F - 1; j >= 0; j--) {
            const int i = f * F + j;
            float vf[VEC], gkf[VEC], gvf[VEC];
            IO::unpack(vr[i], vf);
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                // the bonus term gr e c (v - y) is the token's own part of
                // gk and its whole gu
                const float e = te[i][q];
                const float ed = grt[j][q] * (e * c[q]);
                const float own = ed * (vf[q] - yt[j][q]);
                gvf[q] = __builtin_fmaf(e, S[q], ed);
                gkf[q] = __builtin_fmaf(e, __builtin_fmaf(vf[q], S[q], -SQ[q]), own);
                gu[q] += own;
                gw[q] = __builtin_fmaf(-e, __builtin_fmaf(vf[q], S2[q], -SQ2[q]), gw[q]);
                S2[q] += S[q];
                SQ2[q] += SQ[q];
                S[q] += grt[j][q];
                SQ[q] = __builtin_fmaf(grt[j][q], yt[j][q], SQ[q]);
            }
            Buf<Raw>::template store<kNonTemporalStore>(IO::pack(gkf), gkr_, voff, uint32_t(i) * row_bytes);
            Buf<Raw>::template store<kNonTemporalStore>(IO::pack(gvf), gvr_, voff, uint32_t(i) * row_bytes);
        }
    }
    return true;
}

// Per-lane constants of the backward walk, passed by value.
template <int VEC>
struct Lanes {
    float w[VEC], u[VEC], c[VEC];  // decay, bonus, e^{u-w}
    uint32_t voff, row_bytes;      // byte offset of this lane's channels, of one token
    int lane;
};

// The reverse sums' hand-off through LDS: wait for the carry after
// sub-chunk sc (wave order j), read it into r and pass carry (+) partial on
// to the sub-chunk before.  s_rc holds six rows (P, Q, R, U, Pi, n) of 64 VEC
// floats.
template <int VEC>
__device__ __forceinline__ void rev_handoff(float* s_rc, int* s_rseq, const Lanes<VEC>& ln,
                                            const RState (&rg)[VEC], RState (&r)[VEC], int64_t j,
                                            int64_t sc, int n) {
    constexpr int CG = 64 * VEC;
    while (__hip_atomic_load(s_rseq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != int(j))
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        const int x = ln.lane * VEC + q;
        r[q].P = s_rc[0 * CG + x];
        r[q].Q = s_rc[1 * CG + x];
        r[q].R = s_rc[2 * CG + x];
        r[q].U = s_rc[3 * CG + x];
        r[q].Pi = s_rc[4 * CG + x];
        r[q].n = s_rc[5 * CG + x];
    }
    if (sc > 0) {
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            const int x = ln.lane * VEC + q;
            RState nr = r[q];
            combine_reverse(nr, rg[q], float(n), ln.w[q]);
            s_rc[0 * CG + x] = nr.P;
            s_rc[1 * CG + x] = nr.Q;
            s_rc[2 * CG + x] = nr.R;
            s_rc[3 * CG + x] = nr.U;
            s_rc[4 * CG + x] = nr.Pi;
            s_rc[5 * CG + x] = nr.n;
        }
        if (ln.lane == 0)
            __hip_atomic_store(s_rseq, int(j + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

// The checkpoint (state before the sub-chunk) of this lane's channels, from
// its saved form (r, q): (a, b, A, m) = (r, 1, q, 0), or the empty history.
template <int VEC>
__device__ __forceinline__ void load_checkpoint(FState (&s)[VEC], const float* ck, int64_t C) {
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        from_saved(ck[0 * C + q], ck[1 * C + q], s[q].a, s[q].b, s[q].A);
        s[q].m = 0.0f;
    }
}

// A carry taken by the hand-off, kept in LDS (six rows of 64 per channel).
constexpr int kKeepRows = 6;
template <int VEC>
__device__ __forceinline__ void keep_carry(float* slot, int lane, const RState (&r)[VEC]) {
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        float* o = slot + q * kKeepRows * 64 + lane;
        o[0 * 64] = r[q].P;
        o[1 * 64] = r[q].Q;
        o[2 * 64] = r[q].R;
        o[3 * 64] = r[q].U;
        o[4 * 64] = r[q].Pi;
        o[5 * 64] = r[q].n;
    }
}
template <int VEC>
__device__ __forceinline__ void take_carry(const float* slot, int lane, RState (&r)[VEC]) {
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        const float* o = slot + q * kKeepRows * 64 + lane;
        r[q].P = o[0 * 64];
        r[q].Q = o[1 * 64];
        r[q].R = o[2 * 64];
        r[q].U = o[3 * 64];
        r[q].Pi = o[4 * 64];
        r[q].n = o[5 * 64];
    }
}

template <int VEC>
struct GradWU {
    float gw[VEC], gu[VEC];
};

// One sub-chunk token by token: the forward re-run from the checkpoint, the
// partial of the reverse sums and the hand-off (unless the carry was already
// taken and kept in `slot`), the walk backwards.  Returns the sub-chunk's gw,
// gu terms.
template <typename IO, int L, int VEC, bool FUSED, int LOAD>
__device__ __forceinline__ GradWU<VEC> token_subchunk(const char* kb, const char* vb, const char* gyb,
                                                      char* gkb, char* gvb, const float* ck, int64_t C,
                                                      Lanes<VEC> ln, int n, int64_t j, int64_t sc,
                                                      float* s_rc, int* s_rseq, const float* slot,
                                                      bool have_carry) {
    using Raw = typename IO::Raw;
    const rsrc_t kr_ = make_rsrc(kb);
    const rsrc_t vr_ = make_rsrc(vb);
    const rsrc_t gr_ = make_rsrc(gyb);
    Raw kr[L], vr[L], gyr[L];
#pragma unroll
    for (int i = 0; i < L; i++) {
        if (i < n) {
            const uint32_t o = ln.voff + uint32_t(i) * ln.row_bytes;
            kr[i] = Buf<Raw>::template load<LOAD>(kr_, o, 0);
            vr[i] = Buf<Raw>::template load<LOAD>(vr_, o, 0);
            gyr[i] = Buf<Raw>::template load<LOAD>(gr_, o, 0);
        }
    }
    FState s[VEC];
    load_checkpoint(s, ck, C);
    GradWU<VEC> g;
#pragma unroll
    for (int q = 0; q < VEC; q++) g.gw[q] = g.gu[q] = 0.0f;
    TokenOut to[L][VEC];
    forward_run<IO, L, VEC, FUSED>(s, kr, vr, gyr, ln.w, ln.u, ln.c, n, to, g.gu);
    RState r[VEC];
    if (have_carry) {
        take_carry(slot, ln.lane, r);
    } else {
        // the sub-chunk's partial, max then sum: token i's term has exponent
        // -q_i - i w at the sub-chunk's start and lies i past it
        RState rg[VEC];
        float mx[VEC];
#pragma unroll
        for (int q = 0; q < VEC; q++) mx[q] = kEmptyP;
#pragma unroll
        for (int i = 0; i < L; i++)
            if (i < n)
#pragma unroll
                for (int q = 0; q < VEC; q++)
                    mx[q] = max_num(mx[q], __builtin_fmaf(-float(i), ln.w[q], -to[i][q].q));
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
                    const float xi = __builtin_fmaf(-float(i), ln.w[q], -to[i][q].q);
                    const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(xi, kLog2e, -mxl[q])) * to[i][q].gr;
                    const float ty = t * to[i][q].y;
                    rg[q].P += t;
                    rg[q].Q += ty;
                    rg[q].R = __builtin_fmaf(float(i), t, rg[q].R);
                    rg[q].U = __builtin_fmaf(float(i), ty, rg[q].U);
                }
            }
        }
        rev_handoff(s_rc, s_rseq, ln, rg, r, j, sc, n);
    }
    // the walk backwards from the carry r after the sub-chunk
    const rsrc_t gkr_ = make_rsrc(gkb);
    const rsrc_t gvr_ = make_rsrc(gvb);
#pragma unroll
    for (int i = L - 1; i >= 0; i--) {
        if (i < n) {
            float kf[VEC], vf[VEC], gkf[VEC], gvf[VEC];
            IO::unpack(kr[i], kf);
            IO::unpack(vr[i], vf);
#pragma unroll
            for (int q = 0; q < VEC; q++)
                reverse_detail(r[q], to[i][q], kf[q], vf[q], ln.w[q], i > 0, gkf[q], gvf[q], g.gw[q]);
            const uint32_t o = ln.voff + uint32_t(i) * ln.row_bytes;
            Buf<Raw>::template store<kNonTemporalStore>(IO::pack(gkf), gkr_, o, 0);
            Buf<Raw>::template store<kNonTemporalStore>(IO::pack(gvf), gvr_, o, 0);
        }
    }
    return g;
}

// The same as a call of its own, for the frame loop's fallback: inlined
// there, its registers and the frame path's would be allocated as one.
template <typename IO, int L, int VEC, bool FUSED, int LOAD>
__device__ __attribute__((noinline)) GradWU<VEC> token_subchunk_call(
    const char* kb, const char* vb, const char* gyb, char* gkb, char* gvb, const float* ck, int64_t C,
    Lanes<VEC> ln, int n, int64_t j, int64_t sc, float* s_rc, int* s_rseq, const float* slot,
    bool have_carry) {
    return token_subchunk<IO, L, VEC, FUSED, LOAD>(kb, vb, gyb, gkb, gvb, ck, C, ln, n, j, sc, s_rc, s_rseq,
                                             slot, have_carry);
}

// SAVED: the checkpoints come from the forward that produced y (pr.ckpt holds
// them) and phase F is skipped.
template <int DT, int VEC, int NWV, bool SAVED>
__global__ __launch_bounds__(NWV * 64) void backward_chained_kernel(BackwardProblem pr, int64_t gpr,
                                                                    int64_t nsub) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int L = kBwdTokens;
    constexpr int CG = 64 * VEC;
    // cache policy of phase R's k, v, gy loads: non-temporal when they are
    // read once (saved states); when phase F has read k and v already, the
    // default policy, so that the second reading can hit the caches (bf16
    // workload: 439 -> 431-433 us)
    constexpr int kWalkLoad = SAVED ? kStreamLoad : kDefaultLoad;
    __shared__ float s_fc[4][CG];  // forward carry (a, b, A, m) before sub-chunk s_fseq
    __shared__ float s_rc[6][CG];            // reverse carry after sub-chunk nsub-1-s_rseq
    __shared__ float s_red[2][NWV][CG];      // per-wave gw, gu
    __shared__ int s_fseq, s_rseq;
    // y, gy / den of the frame path's sub-chunk, per wave (two channels a lane)
    constexpr bool STASH = VEC == 2;
    __shared__ float4 s_stash[STASH ? NWV : 1][STASH ? L * 64 : 1];
    // a carry the frame path has taken but could not use, per wave (in the
    // stash, free by then, when there is one)
    __shared__ float s_keep[STASH ? 1 : NWV][STASH ? 1 : kKeepRows * VEC * 64];

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
        // lanes past the last channel mirror lane 0 (its channels' data,
        // parameters and checkpoints): they compute its values bit for bit, so
        // their gk, gv stores write lane 0's bytes once more and need no
        // branch; the range checks still ask only lanes that hold a channel
        w[q] = pr.w[(active ? c : c0) + q];
        u[q] = pr.u[(active ? c : c0) + q];
        const float wmu = w[q] - u[q];
        fus = fus && __builtin_fabsf(wmu) <= kFusedMaxAbsUW;
        cb[q] = __builtin_amdgcn_exp2f(-wmu * kLog2e);  // e^{u-w}
    }
    const bool fused = __builtin_amdgcn_ballot_w64(!fus) == 0;
    bool nar = true;
#pragma unroll
    for (int q = 0; q < VEC; q++) nar = nar && __builtin_fabsf(w[q] - u[q]) <= kNarrowMaxAbsUW;
    const bool narrow = __builtin_amdgcn_ballot_w64(!nar) == 0;
    if (wave == 0) {
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            FState e;
            e.set_empty();
            s_fc[0][lane * VEC + q] = e.a;
            s_fc[1][lane * VEC + q] = e.b;
            s_fc[2][lane * VEC + q] = e.A;
            s_fc[3][lane * VEC + q] = e.m;
            RState r;
            r.set_empty();
            s_rc[0][lane * VEC + q] = r.P;
            s_rc[1][lane * VEC + q] = r.Q;
            s_rc[2][lane * VEC + q] = r.R;
            s_rc[3][lane * VEC + q] = r.U;
            s_rc[4][lane * VEC + q] = r.Pi;
            s_rc[5][lane * VEC + q] = r.n;
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
    // token i of a sub-chunk at byte voff + i row_bytes of its base: the
    // second part as the buffer instructions' scalar offset, so that no
    // vector register holds a per-token offset
    const int64_t gbase = (bb * T * C + c0) * es;
    // checkpoints: [B][nsub][r, q][C] fp32
    // (lanes past the last channel read the group's first channel's)
    float* ckpt = pr.ckpt + bb * nsub * kCkptFields * C + (active ? c : c0);

    // ---------------- phase F: forward carries and checkpoints ----------------
    for (int64_t sc = SAVED ? nsub : wave; sc < nsub; sc += NWV) {
        const int64_t t0 = sc * L;
        const int n = T - t0 >= L ? L : int(T - t0);
        const int64_t base = gbase + t0 * int64_t(row_bytes);
        const rsrc_t kr_ = make_rsrc(static_cast<const char*>(pr.k) + base);
        const rsrc_t vr_ = make_rsrc(static_cast<const char*>(pr.v) + base);
        Raw kr[L], vr[L];
#pragma unroll
        for (int i = 0; i < L; i++) {
            if (i < n) {
                // default policy: phase R reads k and v again (kWalkLoad)
                kr[i] = Buf<Raw>::template load<kDefaultLoad>(kr_, voff, uint32_t(i) * row_bytes);
                vr[i] = Buf<Raw>::template load<kDefaultLoad>(vr_, voff, uint32_t(i) * row_bytes);
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
#pragma unroll
                    for (int q = 0; q < VEC; q++) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[i][q], kLog2e, -mxl[q]));
                        g[q].a = __builtin_fmaf(e, vf[q], g[q].a);
                        g[q].b += e;
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
            x[q].A = s_fc[2][lane * VEC + q];
            x[q].m = s_fc[3][lane * VEC + q];
        }
        if (sc + 1 < nsub) {
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                FState nx = x[q];
                combine_forward(nx, g[q], float(n), w[q]);
                s_fc[0][lane * VEC + q] = nx.a;
                s_fc[1][lane * VEC + q] = nx.b;
                s_fc[2][lane * VEC + q] = nx.A;
                s_fc[3][lane * VEC + q] = nx.m;
            }
            if (lane == 0)
                __hip_atomic_store(&s_fseq, int(sc + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (active) {
            // non-temporal stores, as the forward's saved states (read once),
            // through plain pointers like phase R's loads of them: memory a
            // kernel reads back goes through one kind of access (the
            // matrix-state step's in-place state, read through plain pointers
            // and written through a buffer descriptor, came out
            // nondeterministic; both through the descriptor, it did not)
            float* ck = ckpt + sc * kCkptFields * C;
#pragma unroll
            for (int q = 0; q < VEC; q++) {
                float r, qs;
                to_saved(x[q].a, x[q].b, __builtin_fmaf(-x[q].m, w[q], x[q].A), r, qs);
                store_stream(ck + 0 * C + q, r);
                store_stream(ck + 1 * C + q, qs);
            }
        }
    }
    // every checkpoint is written (and visible to the workgroup) past here
    __syncthreads();

    // ---------------- phase R: the backward walk ----------------
    float gw[VEC], gu[VEC];
#pragma unroll
    for (int q = 0; q < VEC; q++) gw[q] = gu[q] = 0.0f;
    Lanes<VEC> ln;
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        ln.w[q] = w[q];
        ln.u[q] = u[q];
        ln.c[q] = cb[q];
    }
    ln.voff = voff;
    ln.row_bytes = row_bytes;
    ln.lane = lane;
    float* rc = &s_rc[0][0];
    // a carry the frame path has taken but could not use: in the stash (free
    // by then) when there is one
    float* slot;
    if constexpr (STASH)
        slot = reinterpret_cast<float*>(s_stash[wave]);
    else
        slot = s_keep[wave];
    // sub-chunk sc in wave order j: its bases
    auto at = [&](const void* p, int64_t sc) __attribute__((always_inline)) {
        return static_cast<const char*>(p) + gbase + sc * L * int64_t(row_bytes);
    };
    auto at_out = [&](void* p, int64_t sc) __attribute__((always_inline)) {
        return static_cast<char*>(p) + gbase + sc * L * int64_t(row_bytes);
    };
    auto add = [&](const GradWU<VEC>& g) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            gw[q] += g.gw[q];
            gu[q] += g.gu[q];
        }
    };
    // the read-out form is uniform over the workgroup (its waves share the
    // channels): one copy of the loop per form keeps their registers apart
    if (fused && narrow) {
        // frame weights for full sub-chunks; the others, and sub-chunks whose
        // values leave the frames' range, token by token through a call
        for (int64_t j = wave; j < nsub; j += NWV) {
            const int64_t sc = nsub - 1 - j;
            const int64_t t0 = sc * L;
            const int n = T - t0 >= L ? L : int(T - t0);
            const float* ck = ckpt + sc * kCkptFields * C;
            bool have_carry = false;  // the hand-off has run
            if (n == L) {
                Raw kr[L], vr[L], gyr[L];
                {
                    const rsrc_t kr_ = make_rsrc(at(pr.k, sc));
                    const rsrc_t vr_ = make_rsrc(at(pr.v, sc));
                    const rsrc_t gr_ = make_rsrc(at(pr.gy, sc));
#pragma unroll
                    for (int i = 0; i < L; i++) {
                        kr[i] = Buf<Raw>::template load<kWalkLoad>(kr_, voff, uint32_t(i) * row_bytes);
                        vr[i] = Buf<Raw>::template load<kWalkLoad>(vr_, voff, uint32_t(i) * row_bytes);
                        gyr[i] = Buf<Raw>::template load<kWalkLoad>(gr_, voff, uint32_t(i) * row_bytes);
                    }
                }
                FState s[VEC];
                load_checkpoint(s, ck, C);
                float te[L][VEC];
                FrameStore<VEC, STASH> st;
                if constexpr (STASH) {
                    st.p = s_stash[wave];
                    st.lane = lane;
                }
                float G[kBwdFrames][VEC], rho[kBwdFrames][VEC], gwt[VEC], gut[VEC];
                RState rg[VEC];
                if (frames_rerun<IO, L, VEC>(s, kr, vr, gyr, w, cb, te, st, G, rho, rg, active)) {
                    RState r[VEC];
                    rev_handoff(rc, &s_rseq, ln, rg, r, j, sc, n);
                    const rsrc_t gkr_ = make_rsrc(at_out(pr.gk, sc));
                    const rsrc_t gvr_ = make_rsrc(at_out(pr.gv, sc));
                    if (frames_walk<IO, L, VEC>(r, te, st, G, rho, vr, w, cb, gkr_, gvr_, voff, row_bytes, active, gwt,
                                                gut)) {
#pragma unroll
                        for (int q = 0; q < VEC; q++) {
                            gw[q] += gwt[q];
                            gu[q] += gut[q];
                        }
                        continue;
                    }
                    // the carried-in sums overflow: the walk token by token
                    // from the kept carry
                    keep_carry(slot, lane, r);
                    have_carry = true;
                }
            }
            add(token_subchunk_call<IO, L, VEC, true, kWalkLoad>(at(pr.k, sc), at(pr.v, sc), at(pr.gy, sc),
                                                      at_out(pr.gk, sc), at_out(pr.gv, sc), ck, C, ln, n,
                                                      j, sc, rc, &s_rseq, slot, have_carry));
        }
    } else if (fused) {
        for (int64_t j = wave; j < nsub; j += NWV) {
            const int64_t sc = nsub - 1 - j;
            const int64_t t0 = sc * L;
            const int n = T - t0 >= L ? L : int(T - t0);
            add(token_subchunk<IO, L, VEC, true, kWalkLoad>(at(pr.k, sc), at(pr.v, sc), at(pr.gy, sc),
                                                 at_out(pr.gk, sc), at_out(pr.gv, sc),
                                                 ckpt + sc * kCkptFields * C, C, ln, n, j, sc, rc,
                                                 &s_rseq, slot, false));
        }
    } else {
        for (int64_t j = wave; j < nsub; j += NWV) {
            const int64_t sc = nsub - 1 - j;
            const int64_t t0 = sc * L;
            const int n = T - t0 >= L ? L : int(T - t0);
            add(token_subchunk<IO, L, VEC, false, kWalkLoad>(at(pr.k, sc), at(pr.v, sc), at(pr.gy, sc),
                                                  at_out(pr.gk, sc), at_out(pr.gv, sc),
                                                  ckpt + sc * kCkptFields * C, C, ln, n, j, sc, rc,
                                                  &s_rseq, slot, false));
        }
    }

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

size_t backward_workspace_bytes(int64_t B, int64_t T, int64_t C, bool saved) {
    const size_t nsub = size_t((T + kBwdTokens - 1) / kBwdTokens);
    const size_t cols = size_t(B) * size_t(C);
    return (saved ? 0 : up256(cols * nsub * kCkptFields * 4)) + 2 * up256(cols * 4);
}

hipError_t launch_backward(BackwardProblem pr, void* workspace, hipStream_t stream) {
    if (pr.T == 0) {
        hipLaunchKernelGGL(zero_pair, dim3(unsigned((pr.C + 255) / 256)), dim3(256), 0, stream, pr.gw,
                           pr.gu, pr.C);
        return hipGetLastError();
    }
    const int64_t cols = pr.B * pr.C;
    const int64_t nsub = (pr.T + kBwdTokens - 1) / kBwdTokens;
    const bool saved = pr.saved != nullptr;
    char* ws = static_cast<char*>(workspace);
    const size_t ck = saved ? 0 : up256(size_t(cols) * size_t(nsub) * kCkptFields * 4);
    // the kernel only reads the checkpoints when they are saved ones
    pr.ckpt = saved ? const_cast<float*>(pr.saved) : reinterpret_cast<float*>(ws);
    pr.part_w = reinterpret_cast<float*>(ws + ck);
    pr.part_u = reinterpret_cast<float*>(ws + ck + up256(size_t(cols) * 4));
    const int64_t cg = 64 * pr.vec;
    const int64_t gpr = (pr.C + cg - 1) / cg;
    const dim3 grid(unsigned(pr.B * gpr));
    constexpr int NW = 8;
    const dim3 block(NW * 64);
    auto go = [&](auto saved_tag) {
        constexpr bool S = decltype(saved_tag)::value;
        if (pr.dtype == kBF16 && pr.vec == 2)
            hipLaunchKernelGGL((backward_chained_kernel<kBF16, 2, NW, S>), grid, block, 0, stream, pr, gpr, nsub);
        else if (pr.dtype == kBF16)
            hipLaunchKernelGGL((backward_chained_kernel<kBF16, 1, NW, S>), grid, block, 0, stream, pr, gpr, nsub);
        else
            hipLaunchKernelGGL((backward_chained_kernel<kF32, 1, NW, S>), grid, block, 0, stream, pr, gpr, nsub);
    };
    if (saved)
        go(std::integral_constant<bool, true>{});
    else
        go(std::integral_constant<bool, false>{});
    hipLaunchKernelGGL(backward_reduce, dim3(unsigned((pr.C + 255) / 256)), dim3(256), 0, stream, pr);
    return hipGetLastError();
}

}  // namespace wkv
