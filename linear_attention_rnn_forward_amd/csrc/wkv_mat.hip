// Matrix-valued state WKV of RWKV-5 "Eagle" and RWKV-6 "Finch" ([vanos] =
// vanos001.github.io "RWKV (Attention-RNN Hybrid)", the table "Versions:
// RWKV-4 -> Eagle -> Finch" and the matrix-form recurrence under it).  Per
// batch row and head, head dimension 64, state S in R^{64x64} (row i: key
// channel, column j: value channel):
//
//   S_t = diag(d_t) S_{t-1} + k_t v_t^T,    y_t = r_t^T S_t,
//   d_t = exp(-softplus(z_t)),  z_t = a.b + w (the table's decay argument;
//                                per token for Finch, per channel for Eagle)
//
// Forward (training / prefill form): one workgroup of 4 waves per (batch row,
// head); wave w owns value columns [16w, 16w + 16) of the state, which stays
// in fp32 registers in the accumulator layout of a 16x16 MFMA tile (lane l
// holds rows 4(l/16) .. 4(l/16)+3 of column l%16 of each of the four 16-row
// blocks).  The tokens are taken in chunks of 16.  With Lam_t[i] the sum of
// log d over the chunk's tokens up to and including t, the recurrence
// unrolls over a chunk into
//
//   y_t = (r_t e^{Lam_t})^T S_0 + sum_{s<=t} [sum_i r_t[i] e^{Lam_t[i]} k_s[i] e^{-Lam_s[i]}] v_s
//   S_16 = diag(e^{Lam_15}) S_0 + sum_s (k_s e^{Lam_15 - Lam_s}) v_s^T
//
// and every sum over i or s is a dense 16x16x16 product on the matrix cores
// (bf16 operands, fp32 accumulation): the read-out of the carried state, the
// chunk's score matrix, its application to the values, and the state update.
// The factor e^{-Lam_s} is bounded by the chunk's total decay span; a chunk in
// which some channel's span exceeds kSpanMax (a decay of e^{-80} within 16
// tokens) is run token by token instead, on the same registers, in fp32.  fp32
// storage always takes that exact token-by-token form.
//
// Decode step: one wave per (row, head); lane j holds column j of the state,
// which is read, updated and written once: an HBM stream of 8 bytes per state
// element and token.
#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

constexpr int kN = 64;            // head dimension (the page's)
constexpr int kCT = 16;           // tokens per chunk
constexpr float kSpanMax = 80.0f; // largest -Lam_15 of a chunk for the factorised form
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kRowPad = kN + 4;   // bf16 row stride of [token][channel] tiles in LDS
constexpr int kColPad = kCT + 4;  // bf16 row stride of [channel][token] tiles in LDS

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int mat_wave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int mat_lane() { return threadIdx.x & 63; }

// -softplus(z) = -(max(z, 0) + log1p(e^{-|z|})), with log1p(x) = ln(u) x / (u - 1)
// for u = 1 + x != 1 (a few ulp where a plain ln(1 + x) would lose x).
__device__ __forceinline__ float neg_softplus(float z) {
    const float x = __builtin_amdgcn_exp2f(-__builtin_fabsf(z) * kLog2e);
    const float u = 1.0f + x;
    const float l = u == 1.0f ? x
                              : __builtin_amdgcn_logf(u) * kLn2 * x * __builtin_amdgcn_rcpf(u - 1.0f);
    return -(max_num(z, 0.0f) + l);
}

__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// x + (x of the lane n below, within the 16-lane row; 0 for the first n lanes)
template <int SH>
__device__ __forceinline__ float row_shr_add(float x) {
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | SH, 0xf, 0xf, false);
    return x + __int_as_float(y);
}

// inclusive prefix sum over the 16 lanes of each row
__device__ __forceinline__ float row_scan(float x) {
    x = row_shr_add<1>(x);
    x = row_shr_add<2>(x);
    x = row_shr_add<4>(x);
    x = row_shr_add<8>(x);
    return x;
}

// value of lane 15 of this lane's row
__device__ __forceinline__ float row_last(float x) {
    const int src = (mat_lane() | 15) << 2;
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(x)));
}

__device__ __forceinline__ uint32_t bf16_word(float lo, float hi) { return pack_bf16x2(lo, hi); }

__device__ __forceinline__ short4_t pack4(float a, float b, float c, float d) {
    const uint2 u = make_uint2(bf16_word(a, b), bf16_word(c, d));
    return __builtin_bit_cast(short4_t, u);
}

__device__ __forceinline__ short4_t lds4(const uint16_t* p) {
    return __builtin_bit_cast(short4_t, *reinterpret_cast<const uint2*>(p));
}

__device__ __forceinline__ float4_t mfma16(short4_t a, short4_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Four consecutive channels of one token in storage type DT.
template <int DT>
struct Quad;
template <>
struct Quad<kF32> {
    using Raw = float4;
    static __device__ __forceinline__ Raw load(const void* base, int64_t e) {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + e);
    }
    static __device__ __forceinline__ void unpack(Raw r, float (&x)[4]) { x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w; }
    static __device__ __forceinline__ void store(void* base, int64_t e, const float (&x)[4]) {
        *reinterpret_cast<float4*>(static_cast<float*>(base) + e) = make_float4(x[0], x[1], x[2], x[3]);
    }
    static __device__ __forceinline__ Raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};
template <>
struct Quad<kBF16> {
    using Raw = uint2;
    static __device__ __forceinline__ Raw load(const void* base, int64_t e) {
        return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + e);
    }
    static __device__ __forceinline__ void unpack(Raw r, float (&x)[4]) {
        x[0] = __uint_as_float(r.x << 16); x[1] = __uint_as_float(r.x & 0xffff0000u);
        x[2] = __uint_as_float(r.y << 16); x[3] = __uint_as_float(r.y & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(void* base, int64_t e, const float (&x)[4]) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + e) =
            make_uint2(bf16_word(x[0], x[1]), bf16_word(x[2], x[3]));
    }
    static __device__ __forceinline__ Raw zero() { return make_uint2(0u, 0u); }
};

template <int DT>
__device__ __forceinline__ float load_one(const void* base, int64_t e) {
    if constexpr (DT == kF32) return static_cast<const float*>(base)[e];
    else return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[e]) << 16);
}
template <int DT>
__device__ __forceinline__ void store_one(void* base, int64_t e, float x) {
    if constexpr (DT == kF32) static_cast<float*>(base)[e] = x;
    else static_cast<uint16_t*>(base)[e] = uint16_t(bf16_word(x, 0.0f) & 0xffffu);
}

struct MatShared {
    // factorised-form operands, double-buffered by chunk parity
    uint16_t rq[2][kCT][kRowPad];   // r_t[i] e^{Lam_t[i]}
    uint16_t kq[2][kCT][kRowPad];   // k_s[i] e^{-Lam_s[i]}
    uint16_t kdt[2][kN][kColPad];   // k_s[i] e^{Lam_15[i] - Lam_s[i]}, [i][s]
    uint16_t vt[2][kN][kColPad];    // v_s[j], [j][s]
    float el[2][kN];                // e^{Lam_15[i]}
    // token-by-token form: r, k, d, v of the chunk in fp32
    float rf[kCT][kN], kf[kCT][kN], df[kCT][kN], vf[kCT][kN];
    int exact_chunk;                // index of the last chunk that must run token by token
};

// The inputs of one thread for one chunk: four channels of one token.
template <int DT>
struct ChunkIn {
    typename Quad<DT>::Raw r, k, v, z;
};

template <int DT, bool PER_TOKEN_Z>
__device__ __forceinline__ void load_chunk(ChunkIn<DT>& in, const MatProblem& pr, int64_t e, bool live) {
    using Q = Quad<DT>;
    if (live) {
        in.r = Q::load(pr.r, e);
        in.k = Q::load(pr.k, e);
        in.v = Q::load(pr.v, e);
        if constexpr (PER_TOKEN_Z) in.z = Q::load(pr.z, e);
    } else {
        in.r = Q::zero();
        in.k = Q::zero();
        in.v = Q::zero();
        if constexpr (PER_TOKEN_Z) in.z = Q::zero();
    }
}

template <int DT, bool PER_TOKEN_Z, bool EXACT_ONLY>
__global__ __launch_bounds__(256) void mat_forward_kernel(MatProblem pr) {
    using Q = Quad<DT>;
    __shared__ MatShared sh;
    const int wave = mat_wave();
    const int lane = mat_lane();
    const int64_t H = pr.H, T = pr.T, C = H * kN;
    const int64_t bb = blockIdx.x / H;
    const int64_t h = blockIdx.x - bb * H;

    // phase-1 role: token tt of the chunk, channels i0 .. i0+3
    const int tt = lane & 15;
    const int i0 = 4 * (4 * wave + (lane >> 4));
    // matrix-core role: lane group g, column nn of the wave's 16 value columns
    const int g = lane >> 4;
    const int nn = lane & 15;
    const int jcol = 16 * wave + nn;

    // state: S[b][r] = S[16b + 4g + r][jcol]
    float S[4][4];
    const int64_t sbase = (bb * H + h) * int64_t(kN * kN);
#pragma unroll
    for (int b = 0; b < 4; b++)
#pragma unroll
        for (int r = 0; r < 4; r++)
            S[b][r] = pr.s_in ? pr.s_in[sbase + int64_t(16 * b + 4 * g + r) * kN + jcol] : 0.0f;

    // per-channel decay (Eagle): log d once
    float lc[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (!PER_TOKEN_Z) {
#pragma unroll
        for (int c = 0; c < 4; c++) lc[c] = neg_softplus(static_cast<const float*>(pr.z)[h * kN + i0 + c]);
    }
    if (threadIdx.x == 0) sh.exact_chunk = -1;

    const int64_t nch = (T + kCT - 1) / kCT;
    const int64_t row0 = bb * T;  // first token row of this batch row
    ChunkIn<DT> nxt;
    if (nch > 0) load_chunk<DT, PER_TOKEN_Z>(nxt, pr, (row0 + tt) * C + h * kN + i0, tt < T);

    for (int64_t ch = 0; ch < nch; ch++) {
        const int64_t t0 = ch * kCT;
        const int n = T - t0 < kCT ? int(T - t0) : kCT;
        const bool live = tt < n;
        const ChunkIn<DT> cur = nxt;
        if (ch + 1 < nch)
            load_chunk<DT, PER_TOKEN_Z>(nxt, pr, (row0 + t0 + kCT + tt) * C + h * kN + i0,
                                        t0 + kCT + tt < T);
        const int buf = int(ch & 1);

        // ---- phase 1: log decay, its prefix over the chunk, operands ----
        float rv[4], kv[4], vv[4], lam[4], lamL[4];
        Q::unpack(cur.r, rv);
        Q::unpack(cur.k, kv);
        Q::unpack(cur.v, vv);
        float lg[4];
        if constexpr (PER_TOKEN_Z) {
            float zv[4];
            Q::unpack(cur.z, zv);
#pragma unroll
            for (int c = 0; c < 4; c++) lg[c] = live ? neg_softplus(zv[c]) : 0.0f;
        } else {
#pragma unroll
            for (int c = 0; c < 4; c++) lg[c] = live ? lc[c] : 0.0f;
        }
#pragma unroll
        for (int c = 0; c < 4; c++) {
            lam[c] = row_scan(lg[c]);
            lamL[c] = row_last(lam[c]);
        }
        if constexpr (!EXACT_ONLY) {
            bool wide = false;
            float rq[4], kq[4], kd[4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
                wide = wide || !(-lamL[c] <= kSpanMax);
                const float ep = exp_f(lam[c]);     // <= 1
                const float en = exp_f(-lam[c]);    // <= e^{span}
                const float eL = exp_f(lamL[c]);
                rq[c] = rv[c] * ep;
                kq[c] = kv[c] * en;
                kd[c] = kv[c] * (eL * en);
                if (tt == 15) sh.el[buf][i0 + c] = eL;
                sh.kdt[buf][i0 + c][tt] = uint16_t(bf16_word(kd[c], 0.0f) & 0xffffu);
                sh.vt[buf][i0 + c][tt] = uint16_t(bf16_word(vv[c], 0.0f) & 0xffffu);
            }
            *reinterpret_cast<uint2*>(&sh.rq[buf][tt][i0]) =
                make_uint2(bf16_word(rq[0], rq[1]), bf16_word(rq[2], rq[3]));
            *reinterpret_cast<uint2*>(&sh.kq[buf][tt][i0]) =
                make_uint2(bf16_word(kq[0], kq[1]), bf16_word(kq[2], kq[3]));
            if (__builtin_amdgcn_ballot_w64(wide) != 0 && lane == 0) sh.exact_chunk = int(ch);
        }
        __syncthreads();
        const bool exact = EXACT_ONLY || sh.exact_chunk == int(ch);

        if (exact) {
            // ---- token by token, fp32 ----
#pragma unroll
            for (int c = 0; c < 4; c++) {
                sh.rf[tt][i0 + c] = rv[c];
                sh.kf[tt][i0 + c] = kv[c];
                sh.df[tt][i0 + c] = exp_f(lg[c]);
                sh.vf[tt][i0 + c] = vv[c];
            }
            __syncthreads();
            for (int t = 0; t < n; t++) {
                const float vj = sh.vf[t][jcol];
                float yp = 0.0f;
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    const float4 d4 = *reinterpret_cast<const float4*>(&sh.df[t][16 * b + 4 * g]);
                    const float4 k4 = *reinterpret_cast<const float4*>(&sh.kf[t][16 * b + 4 * g]);
                    const float4 r4 = *reinterpret_cast<const float4*>(&sh.rf[t][16 * b + 4 * g]);
                    const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
                    const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
                    const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        S[b][r] = __builtin_fmaf(dd[r], S[b][r], kk[r] * vj);
                        yp = __builtin_fmaf(rr[r], S[b][r], yp);
                    }
                }
                // the four lane groups hold the partial sums over disjoint rows
                const float y01 = yp + __shfl_xor(yp, 16);
                const float y = y01 + __shfl_xor(y01, 32);
                if (g == 0) store_one<DT>(pr.y, (row0 + t0 + t) * C + h * kN + jcol, y);
            }
            __syncthreads();
        } else if constexpr (!EXACT_ONLY) {
            // ---- the chunk on the matrix cores ----
            short4_t rqB[4], kqA[4], kdA[4];
#pragma unroll
            for (int b = 0; b < 4; b++) {
                rqB[b] = lds4(&sh.rq[buf][nn][16 * b + 4 * g]);
                kqA[b] = lds4(&sh.kq[buf][nn][16 * b + 4 * g]);
                kdA[b] = lds4(&sh.kdt[buf][16 * b + nn][4 * g]);
            }
            const short4_t vA = lds4(&sh.vt[buf][jcol][4 * g]);
            float4_t yacc = {0.f, 0.f, 0.f, 0.f};
            float4_t aacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < 4; b++) {
                yacc = mfma16(pack4(S[b][0], S[b][1], S[b][2], S[b][3]), rqB[b], yacc);
                aacc = mfma16(kqA[b], rqB[b], aacc);
            }
            // aacc[r] = score of key token s = 4g + r for query token nn; causal mask s <= t
            float am[4];
#pragma unroll
            for (int r = 0; r < 4; r++) am[r] = (4 * g + r <= nn) ? aacc[r] : 0.0f;
            yacc = mfma16(vA, pack4(am[0], am[1], am[2], am[3]), yacc);
            // yacc[r] = y[token nn][column 16 wave + 4g + r]
            if (nn < n) {
                const float yo[4] = {yacc[0], yacc[1], yacc[2], yacc[3]};
                Q::store(pr.y, (row0 + t0 + nn) * C + h * kN + 16 * wave + 4 * g, yo);
            }
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const float4 e4 = *reinterpret_cast<const float4*>(&sh.el[buf][16 * b + 4 * g]);
                float4_t c = {S[b][0] * e4.x, S[b][1] * e4.y, S[b][2] * e4.z, S[b][3] * e4.w};
                c = mfma16(kdA[b], vA, c);
#pragma unroll
                for (int r = 0; r < 4; r++) S[b][r] = c[r];
            }
        }
    }
    if (pr.s_out) {
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                pr.s_out[sbase + int64_t(16 * b + 4 * g + r) * kN + jcol] = S[b][r];
    }
}

// One token for every (row, head): lane j holds column j of the head's state.
template <int DT, bool PER_TOKEN_Z>
__global__ __launch_bounds__(256) void mat_step_kernel(MatStepProblem pr) {
    const int lane = mat_lane();
    const int64_t head = int64_t(blockIdx.x) * 4 + mat_wave();
    const int64_t H = pr.H, C = H * kN;
    if (head >= pr.L * pr.S * H) return;
    const int64_t row = head / H;          // l * S + s
    const int64_t h = head - row * H;
    const int64_t layer = row / pr.S;
    const int64_t e = row * C + h * kN + lane;
    const float r = load_one<DT>(pr.r, e);
    const float k = load_one<DT>(pr.k, e);
    const float v = load_one<DT>(pr.v, e);
    const float z = PER_TOKEN_Z ? load_one<DT>(pr.z, e)
                                : static_cast<const float*>(pr.z)[layer * C + h * kN + lane];
    const float d = exp_f(neg_softplus(z));
    const int64_t sb = head * int64_t(kN * kN) + lane;
    float s[kN];
#pragma unroll
    for (int i = 0; i < kN; i++) s[i] = pr.s_in[sb + i * kN];
    float y = 0.0f;
#pragma unroll
    for (int i = 0; i < kN; i++) {
        // d, k, r of key channel i, from lane i (wave-uniform)
        const float di = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), i));
        const float ki = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k), i));
        const float ri = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), i));
        s[i] = __builtin_fmaf(di, s[i], ki * v);
        y = __builtin_fmaf(ri, s[i], y);
    }
#pragma unroll
    for (int i = 0; i < kN; i++) pr.s_out[sb + i * kN] = s[i];
    store_one<DT>(pr.y, e, y);
}

}  // namespace

hipError_t launch_mat_forward(const MatProblem& pr, hipStream_t stream) {
    const dim3 grid(unsigned(pr.B * pr.H)), block(256);
    const bool exact = pr.dtype == kF32 || pr.path == 1;
#define WKV_MAT_FWD(DT, PT, EX) hipLaunchKernelGGL((mat_forward_kernel<DT, PT, EX>), grid, block, 0, stream, pr)
    if (pr.dtype == kF32) {
        if (pr.z_per_token) WKV_MAT_FWD(kF32, true, true);
        else WKV_MAT_FWD(kF32, false, true);
    } else if (exact) {
        if (pr.z_per_token) WKV_MAT_FWD(kBF16, true, true);
        else WKV_MAT_FWD(kBF16, false, true);
    } else {
        if (pr.z_per_token) WKV_MAT_FWD(kBF16, true, false);
        else WKV_MAT_FWD(kBF16, false, false);
    }
#undef WKV_MAT_FWD
    return hipGetLastError();
}

hipError_t launch_mat_step(const MatStepProblem& pr, hipStream_t stream) {
    const int64_t heads = pr.L * pr.S * pr.H;
    const dim3 grid(unsigned((heads + 3) / 4)), block(256);
#define WKV_MAT_STEP(DT, PT) hipLaunchKernelGGL((mat_step_kernel<DT, PT>), grid, block, 0, stream, pr)
    if (pr.dtype == kF32) {
        if (pr.z_per_token) WKV_MAT_STEP(kF32, true);
        else WKV_MAT_STEP(kF32, false);
    } else {
        if (pr.z_per_token) WKV_MAT_STEP(kBF16, true);
        else WKV_MAT_STEP(kBF16, false);
    }
#undef WKV_MAT_STEP
    return hipGetLastError();
}

}  // namespace wkv
