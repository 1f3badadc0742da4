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
// blocks).  The tokens are taken in chunks of 16.  With D_t[i] the product of
// the decays d[i] of the chunk's tokens up to and including t, the recurrence
// unrolls over a chunk into
//
//   y_t = (r_t D_t)^T S_0 + sum_{s<=t} [sum_i r_t[i] D_t[i] k_s[i] / D_s[i]] v_s
//   S_16 = diag(D_15) S_0 + sum_s (k_s D_15 / D_s) v_s^T
//
// and every sum over i or s is a dense 16x16x16 product on the matrix cores
// (bf16 operands, fp32 accumulation): the read-out of the carried state, the
// chunk's score matrix, its application to the values, and the state update.
// The prefix products run across the 16 lanes of a row with DPP.  The factor
// 1/D_s is bounded by the chunk's total decay; a chunk in which some channel
// decays by more than e^{-80} is run token by token instead, on the same
// registers, in fp32.  fp32 storage always takes that exact token-by-token
// form.
//
// Decode step: one wave per (row, head); each state element is read, updated
// and written once: an HBM stream of 8 bytes per state element and token.
#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

constexpr int kN = 64;            // head dimension (the page's)
constexpr int kCT = 16;           // tokens per chunk
constexpr float kMinChunkDecay = 1.8e-35f;  // e^{-80}: the smallest decay over a chunk that
                                           // the factorised form takes (1/D stays <= e^{80})
constexpr int kRowPad = kN + 4;   // bf16 row stride of [token][channel] tiles in LDS
constexpr int kColPad = kCT + 4;  // bf16 row stride of [channel][token] tiles in LDS

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int mat_wave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int mat_lane() { return threadIdx.x & 63; }

__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// x * (x of the lane SH below, within the 16-lane row), in place: the first
// SH lanes of each row have no source and keep x (v_mul_f32_dpp without
// bound_ctrl leaves such lanes unwritten).  The s_nop covers the two wait
// states a DPP read needs after a vector write of its source.
template <int SH>
__device__ __forceinline__ float row_shr_mul(float x) {
    float y;
    if constexpr (SH == 1)
        asm volatile("s_nop 1\n\tv_mul_f32_dpp %0, %1, %2 row_shr:1 row_mask:0xf bank_mask:0xf"
                     : "=v"(y) : "v"(x), "v"(x), "0"(x));
    else if constexpr (SH == 2)
        asm volatile("s_nop 1\n\tv_mul_f32_dpp %0, %1, %2 row_shr:2 row_mask:0xf bank_mask:0xf"
                     : "=v"(y) : "v"(x), "v"(x), "0"(x));
    else if constexpr (SH == 4)
        asm volatile("s_nop 1\n\tv_mul_f32_dpp %0, %1, %2 row_shr:4 row_mask:0xf bank_mask:0xf"
                     : "=v"(y) : "v"(x), "v"(x), "0"(x));
    else
        asm volatile("s_nop 1\n\tv_mul_f32_dpp %0, %1, %2 row_shr:8 row_mask:0xf bank_mask:0xf"
                     : "=v"(y) : "v"(x), "v"(x), "0"(x));
    return y;
}

// inclusive prefix product over the 16 lanes of each row
__device__ __forceinline__ float row_prod(float x) {
    x = row_shr_mul<1>(x);
    x = row_shr_mul<2>(x);
    x = row_shr_mul<4>(x);
    x = row_shr_mul<8>(x);
    return x;
}

// value of lane 15 of this lane's row (DPP row_newbcast)
__device__ __forceinline__ float row_last(float x) {
    float y;
    asm volatile("s_nop 1\n\tv_mov_b32_dpp %0, %1 row_newbcast:15 row_mask:0xf bank_mask:0xf"
                 : "=v"(y) : "v"(x));
    return y;
}

// d = exp(-softplus(z)) = 1 / (1 + e^z): 1 for z = -inf, 0 once e^z overflows
__device__ __forceinline__ float decay_of(float z) { return __builtin_amdgcn_rcpf(1.0f + exp_f(z)); }


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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// 16x16x32: lane l supplies k = 8(l/16) .. 8(l/16)+7 of its row (A) or column
// (B); the eight values are the two 4-value halves lo, hi.
__device__ __forceinline__ float4_t mfma32(short4_t alo, short4_t ahi, short4_t blo, short4_t bhi,
                                           float4_t c) {
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7));
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7));
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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
    // operands of the chunked form, double-buffered by chunk parity
    uint16_t rq[2][kCT][kRowPad];   // r_t[i] D_t[i]
    uint16_t kq[2][kCT][kRowPad];   // k_s[i] / D_s[i]
    uint16_t kdt[2][kN][kColPad];   // k_s[i] D_15[i] / D_s[i], [i][s]
    uint16_t vt[2][kN][kColPad];    // v_s[j], [j][s]
    float el[2][kN];                // D_15[i]
    // fp32 storage (token-by-token form only): r, k, d, v of the chunk, rows
    // padded so that a wave's 16-byte writes spread over the banks
    float rf[2][kCT][kN + 4], kf[2][kCT][kN + 4], df[2][kCT][kN + 4], vf[2][kCT][kN + 4];
    uint16_t yt[2][kCT][kRowPad];   // y of a chunk (chunked form), written out one chunk later
    int exact_chunk[2];             // chunk of this parity that must run token by token
};

// The inputs of one producer thread for one chunk: four channels of one token.
template <int DT>
struct ChunkIn {
    typename Quad<DT>::Raw r, k, v, z;
};

// Unconditional loads (a branch around them would make every later use wait
// for all outstanding loads); the caller clamps the token to a valid one and
// masks the padding tokens afterwards.
template <int DT, bool PER_TOKEN_Z>
__device__ __forceinline__ void load_chunk(ChunkIn<DT>& in, const MatProblem& pr, int64_t e) {
    using Q = Quad<DT>;
    in.r = Q::load(pr.r, e);
    in.k = Q::load(pr.k, e);
    in.v = Q::load(pr.v, e);
    if constexpr (PER_TOKEN_Z) in.z = Q::load(pr.z, e);
}

__device__ __forceinline__ float4 keep_if(bool live, float4 x) {
    return live ? x : make_float4(0.f, 0.f, 0.f, 0.f);
}
__device__ __forceinline__ uint2 keep_if(bool live, uint2 x) { return live ? x : make_uint2(0u, 0u); }
// padding tokens get z = -inf: d = 1, no decay
__device__ __forceinline__ float4 pad_z(bool live, float4 x) {
    const float ni = -__builtin_inff();
    return live ? x : make_float4(ni, ni, ni, ni);
}
__device__ __forceinline__ uint2 pad_z(bool live, uint2 x) {
    return live ? x : make_uint2(0xff80ff80u, 0xff80ff80u);
}

// v_s[j] of four channels of one token into the [channel][token] tile: bf16
// storage is written as stored, fp32 is rounded.
template <int DT>
__device__ __forceinline__ void store_vt(uint16_t (*vt)[kColPad], int i0, int tt,
                                         typename Quad<DT>::Raw raw, const float (&vv)[4]) {
    if constexpr (DT == kBF16) {
        vt[i0 + 0][tt] = uint16_t(raw.x & 0xffffu);
        vt[i0 + 1][tt] = uint16_t(raw.x >> 16);
        vt[i0 + 2][tt] = uint16_t(raw.y & 0xffffu);
        vt[i0 + 3][tt] = uint16_t(raw.y >> 16);
    } else {
#pragma unroll
        for (int c = 0; c < 4; c++) vt[i0 + c][tt] = uint16_t(bf16_word(vv[c], 0.0f) & 0xffffu);
    }
}

__device__ __forceinline__ int chunk_tokens(int64_t T, int64_t ch) {
    const int64_t left = T - ch * kCT;  // <= 0 past the last chunk
    return left < kCT ? (left > 0 ? int(left) : 0) : kCT;
}

// Producer: the operands of chunk ch into LDS buffer ch & 1.  Thread (tt, i0)
// handles token tt of the chunk and channels i0 .. i0+3.  Chunks past the last
// one are all padding (no decay, zero keys).
template <int DT, bool PER_TOKEN_Z, bool EXACT_ONLY>
__device__ __forceinline__ void produce_chunk(MatShared& sh, int tt, int i0, int lane,
                                              const ChunkIn<DT>& cur, const float (&dc)[4],
                                              int64_t T, int64_t ch) {
    using Q = Quad<DT>;
    const int buf = int(ch & 1);
    const bool live = tt < chunk_tokens(T, ch);
    float rv[4], kv[4], vv[4], dcy[4];
    const typename Q::Raw vraw = keep_if(live, cur.v);
    Q::unpack(keep_if(live, cur.r), rv);
    Q::unpack(keep_if(live, cur.k), kv);
    Q::unpack(vraw, vv);
    if constexpr (PER_TOKEN_Z) {
        float zv[4];
        Q::unpack(pad_z(live, cur.z), zv);
#pragma unroll
        for (int c = 0; c < 4; c++) dcy[c] = decay_of(zv[c]);
    } else {
#pragma unroll
        for (int c = 0; c < 4; c++) dcy[c] = live ? dc[c] : 1.0f;
    }
    if constexpr (EXACT_ONLY) {
        // the token-by-token form's inputs
        *reinterpret_cast<float4*>(&sh.rf[buf][tt][i0]) = make_float4(rv[0], rv[1], rv[2], rv[3]);
        *reinterpret_cast<float4*>(&sh.kf[buf][tt][i0]) = make_float4(kv[0], kv[1], kv[2], kv[3]);
        *reinterpret_cast<float4*>(&sh.df[buf][tt][i0]) = make_float4(dcy[0], dcy[1], dcy[2], dcy[3]);
        *reinterpret_cast<float4*>(&sh.vf[buf][tt][i0]) = make_float4(vv[0], vv[1], vv[2], vv[3]);
    } else {
        bool wide = false;
        float rq[4], kq[4];
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const float D = row_prod(dcy[c]);      // D_t = prod_{tau <= t} d_tau, <= 1
            const float DL = row_last(D);          // D_15
            wide = wide || !(DL >= kMinChunkDecay);
            const float inv = __builtin_amdgcn_rcpf(D);   // <= 1 / D_15
            rq[c] = rv[c] * D;
            kq[c] = kv[c] * inv;
            const float kd = kv[c] * (DL * inv);
            if (tt == 15) sh.el[buf][i0 + c] = DL;
            sh.kdt[buf][i0 + c][tt] = uint16_t(bf16_word(kd, 0.0f) & 0xffffu);
        }
        store_vt<DT>(sh.vt[buf], i0, tt, vraw, vv);
        *reinterpret_cast<uint2*>(&sh.rq[buf][tt][i0]) =
            make_uint2(bf16_word(rq[0], rq[1]), bf16_word(rq[2], rq[3]));
        *reinterpret_cast<uint2*>(&sh.kq[buf][tt][i0]) =
            make_uint2(bf16_word(kq[0], kq[1]), bf16_word(kq[2], kq[3]));
        if (__builtin_amdgcn_ballot_w64(wide) != 0 && lane == 0) sh.exact_chunk[buf] = int(ch);
    }
}

// r, k, d of token row e (element offset of its channel 0 in this head) for
// channels c0 .. c0+3, and v of channel jcol, read from global memory (the
// rare token-by-token chunk of the chunked kernel).
template <int DT, bool PER_TOKEN_Z>
__device__ __forceinline__ void token_inputs(const MatProblem& pr, int64_t e, int64_t zc, int c0,
                                             float (&r)[4], float (&k)[4], float (&d)[4]) {
    using Q = Quad<DT>;
    Q::unpack(Q::load(pr.r, e + c0), r);
    Q::unpack(Q::load(pr.k, e + c0), k);
    if constexpr (PER_TOKEN_Z) {
        float z[4];
        Q::unpack(Q::load(pr.z, e + c0), z);
#pragma unroll
        for (int c = 0; c < 4; c++) d[c] = decay_of(z[c]);
    } else {
#pragma unroll
        for (int c = 0; c < 4; c++) d[c] = decay_of(static_cast<const float*>(pr.z)[zc + c0 + c]);
    }
}

// Consumer: chunk ch from LDS buffer ch & 1 against the state S (accumulator
// layout: S[b][r] = S[16b + 4g + r][jcol]).  The token-by-token form writes y
// of its 16 value columns to global memory at once; the chunked form leaves
// it in the tile yt[ch & 1] and returns true (store_tile writes it out).
template <int DT, bool PER_TOKEN_Z, bool EXACT_ONLY>
__device__ __forceinline__ bool consume_chunk(const MatProblem& pr, MatShared& sh, int wave, int g,
                                              int nn, int64_t row0, int64_t h, int64_t ch,
                                              float (&S)[4][4]) {
    using Q = Quad<DT>;
    const int64_t C = pr.H * kN;
    const int64_t t0 = ch * kCT;
    const int n = chunk_tokens(pr.T, ch);
    const int buf = int(ch & 1);
    const int jcol = 16 * wave + nn;
    // The chunked form's operands are read before the choice of form, so that
    // their LDS latency overlaps the flag's (reading them is harmless when the
    // chunk runs token by token).
    short4_t rqB[4], kqA[4], kdA[4], vA;
    if constexpr (!EXACT_ONLY) {
#pragma unroll
        for (int b = 0; b < 4; b++) {
            rqB[b] = lds4(&sh.rq[buf][nn][16 * b + 4 * g]);
            kqA[b] = lds4(&sh.kq[buf][nn][16 * b + 4 * g]);
            kdA[b] = lds4(&sh.kdt[buf][16 * b + nn][4 * g]);
        }
        vA = lds4(&sh.vt[buf][jcol][4 * g]);
    }
    if (EXACT_ONLY || sh.exact_chunk[buf] == int(ch)) {
        // ---- token by token, fp32 ----
        for (int t = 0; t < n; t++) {
            const int64_t e = (row0 + t0 + t) * C + h * kN;
            const float vj = EXACT_ONLY ? sh.vf[buf][t][jcol] : load_one<DT>(pr.v, e + jcol);
            float yp = 0.0f;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                float dd[4], kk[4], rr[4];
                if constexpr (EXACT_ONLY) {
                    const float4 d4 = *reinterpret_cast<const float4*>(&sh.df[buf][t][16 * b + 4 * g]);
                    const float4 k4 = *reinterpret_cast<const float4*>(&sh.kf[buf][t][16 * b + 4 * g]);
                    const float4 r4 = *reinterpret_cast<const float4*>(&sh.rf[buf][t][16 * b + 4 * g]);
                    dd[0] = d4.x; dd[1] = d4.y; dd[2] = d4.z; dd[3] = d4.w;
                    kk[0] = k4.x; kk[1] = k4.y; kk[2] = k4.z; kk[3] = k4.w;
                    rr[0] = r4.x; rr[1] = r4.y; rr[2] = r4.z; rr[3] = r4.w;
                } else {
                    token_inputs<DT, PER_TOKEN_Z>(pr, e, h * kN, 16 * b + 4 * g, rr, kk, dd);
                }
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    S[b][r] = __builtin_fmaf(dd[r], S[b][r], kk[r] * vj);
                    yp = __builtin_fmaf(rr[r], S[b][r], yp);
                }
            }
            // the four lane groups hold the partial sums over disjoint rows
            const float y01 = yp + __shfl_xor(yp, 16);
            const float y = y01 + __shfl_xor(y01, 32);
            if (g == 0) store_one<DT>(pr.y, e + jcol, y);
        }
        return false;
    }
    if constexpr (!EXACT_ONLY) {
        // ---- the chunk on the matrix cores ----
        float4_t yacc = {0.f, 0.f, 0.f, 0.f};
        float4_t aacc = {0.f, 0.f, 0.f, 0.f};
        // the contraction over the 64 key channels as two 16x16x32 products:
        // lane group g supplies rows 16b + 4g .. +3 of blocks b = 2m, 2m+1 (its
        // own state registers), and the same channels of rq and kq
#pragma unroll
        for (int m = 0; m < 2; m++) {
            const short4_t s0 = pack4(S[2 * m][0], S[2 * m][1], S[2 * m][2], S[2 * m][3]);
            const short4_t s1 = pack4(S[2 * m + 1][0], S[2 * m + 1][1], S[2 * m + 1][2], S[2 * m + 1][3]);
            yacc = mfma32(s0, s1, rqB[2 * m], rqB[2 * m + 1], yacc);
            aacc = mfma32(kqA[2 * m], kqA[2 * m + 1], rqB[2 * m], rqB[2 * m + 1], aacc);
        }
        // aacc[r] = score of key token s = 4g + r for query token nn; causal mask s <= t
        float am[4];
#pragma unroll
        for (int r = 0; r < 4; r++) am[r] = (4 * g + r <= nn) ? aacc[r] : 0.0f;
        yacc = mfma16(vA, pack4(am[0], am[1], am[2], am[3]), yacc);
        // yacc[r] = y[token nn][column 16 wave + 4g + r], into the tile: a
        // wave's direct stores would write 32 bytes of each of 16 rows
        *reinterpret_cast<uint2*>(&sh.yt[buf][nn][16 * wave + 4 * g]) =
            make_uint2(bf16_word(yacc[0], yacc[1]), bf16_word(yacc[2], yacc[3]));
        // S <- diag(D_15) S + Kd^T V: the product does not wait for D_15
        float4_t upd[4];
#pragma unroll
        for (int b = 0; b < 4; b++) upd[b] = mfma16(kdA[b], vA, float4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const float4 e4 = *reinterpret_cast<const float4*>(&sh.el[buf][16 * b + 4 * g]);
            S[b][0] = __builtin_fmaf(S[b][0], e4.x, upd[b][0]);
            S[b][1] = __builtin_fmaf(S[b][1], e4.y, upd[b][1]);
            S[b][2] = __builtin_fmaf(S[b][2], e4.z, upd[b][2]);
            S[b][3] = __builtin_fmaf(S[b][3], e4.w, upd[b][3]);
        }
    }
    return true;
}

// The y tile of chunk ch (n valid rows) from LDS to global memory in whole
// rows: consumer thread ct writes 4 channels of row ct / 16, so a wave writes
// 4 rows of 128 bytes per instruction.
// (read_tile issues the LDS read early; write_tile stores it once it is needed.)
__device__ __forceinline__ uint2 read_tile(MatShared& sh, int ct, int64_t ch) {
    return *reinterpret_cast<const uint2*>(&sh.yt[ch & 1][ct >> 4][(ct & 15) * 4]);
}
__device__ __forceinline__ void write_tile(const MatProblem& pr, uint2 v, int ct, int64_t row0,
                                           int64_t h, int64_t ch, int n) {
    const int row = ct >> 4;
    if (row < n)
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(pr.y) + (row0 + ch * kCT + row) * pr.H * kN +
                                  h * kN + (ct & 15) * 4) = v;
}
__device__ __forceinline__ void store_tile(const MatProblem& pr, MatShared& sh, int ct,
                                           int64_t row0, int64_t h, int64_t ch, int n) {
    write_tile(pr, read_tile(sh, ct, ch), ct, row0, h, ch, n);
}

// Chunks in flight per producer thread: the inputs of the next kPrefetch
// chunks are loaded into registers while the current one is processed.
constexpr int kPrefetch = 4;

// One workgroup of 8 waves per (batch row, head).  Waves 4..7 produce the
// operands of chunk c+1 while waves 0..3 consume chunk c (matrix-core products
// and the state); one barrier per chunk hands the double-buffered LDS over.
template <int DT, bool PER_TOKEN_Z, bool EXACT_ONLY>
__global__ __launch_bounds__(512, 4) void mat_forward_kernel(MatProblem pr) {
    __shared__ MatShared sh;
    const int wave = mat_wave();
    const int lane = mat_lane();
    const bool producer = wave >= 4;
    const int64_t T = pr.T, C = pr.H * kN;
    const int64_t bb = blockIdx.x / pr.H;
    const int64_t h = blockIdx.x - bb * pr.H;
    const int64_t row0 = bb * T;
    const int64_t nch = (T + kCT - 1) / kCT;
    // producer role: token tt of a chunk, channels i0 .. i0+3
    const int tt = lane & 15;
    const int i0 = 4 * (4 * (wave & 3) + (lane >> 4));
    // consumer role: lane group g, column nn of the wave's 16 value columns
    const int g = lane >> 4;
    const int nn = lane & 15;
    const int jcol = 16 * (wave & 3) + nn;

    float S[4][4];
    const int64_t sbase = (bb * pr.H + h) * int64_t(kN * kN);
    if (!producer) {
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                S[b][r] = pr.s_in ? pr.s_in[sbase + int64_t(16 * b + 4 * g + r) * kN + jcol] : 0.0f;
    }
    // per-channel decay (Eagle): d once
    float dc[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (!PER_TOKEN_Z) {
        if (producer) {
#pragma unroll
            for (int c = 0; c < 4; c++) dc[c] = decay_of(static_cast<const float*>(pr.z)[h * kN + i0 + c]);
        }
    }
    if (threadIdx.x < 2) sh.exact_chunk[threadIdx.x] = -1;
    // the state and decay loads complete here (s_waitcnt vmcnt(0) as an
    // instruction the compiler's wait insertion sees), so that the waits inside
    // the chunk loop only count the prefetch ring's loads
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // element offset of token tt of chunk ch (ch >= 0), clamped to the last
    // token; only called when T >= 1
    const int64_t e0 = row0 * C + h * kN + i0;
    auto elem = [&](int64_t ch) {
        const int64_t t = ch * kCT + tt;
        return e0 + (t < T ? t : T - 1) * C;
    };
    // The producers keep a ring of kPrefetch chunks in registers: slot p is
    // consumed, then reloaded in place with the chunk kPrefetch ahead.  Loads
    // are unconditional (chunks past the last one load the last token; their
    // values are masked as padding).  In the interval of chunk q the producers
    // prepare q while the consumers process q - 1.  The two roles run separate
    // loops (so that neither holds the other's registers) with the same number
    // of barriers; nothing happens for T = 0.
    int64_t pend = -1;  // consumers: chunk whose y tile is still to be written
    if (nch > 0) {
        if (producer) {
            // the first pass only loads (a prologue outside the loop would
            // reach the loop with the slots loaded in another order, and the
            // waits would then cover every load in flight)
            ChunkIn<DT> ring[kPrefetch];
            for (int64_t q0 = -kPrefetch; q0 <= nch; q0 += kPrefetch) {
#pragma unroll
                for (int p = 0; p < kPrefetch; p++) {
                    const int64_t q = q0 + p;
                    if (q0 >= 0) produce_chunk<DT, PER_TOKEN_Z, EXACT_ONLY>(sh, tt, i0, lane, ring[p], dc, T, q);
                    load_chunk<DT, PER_TOKEN_Z>(ring[p], pr, elem(q + kPrefetch));
                    if (q0 >= 0) __syncthreads();
                }
            }
        } else {
            // the y tile of the chunk consumed in the previous interval is
            // written out in this one (after the barrier that completes it)
            for (int64_t q0 = 0; q0 <= nch; q0 += kPrefetch) {
#pragma unroll
                for (int p = 0; p < kPrefetch; p++) {
                    const int64_t q = q0 + p;
                    const int64_t prev = pend;
                    uint2 tile = make_uint2(0u, 0u);
                    if (prev >= 0) tile = read_tile(sh, int(threadIdx.x), prev);
                    pend = -1;
                    if (q >= 1 && q <= nch &&
                        consume_chunk<DT, PER_TOKEN_Z, EXACT_ONLY>(pr, sh, wave, g, nn, row0, h, q - 1, S))
                        pend = q - 1;
                    if (prev >= 0) write_tile(pr, tile, int(threadIdx.x), row0, h, prev, chunk_tokens(T, prev));
                    __syncthreads();
                }
            }
        }
    }
    // both roles: the last tile, if still pending, after one more barrier
    __syncthreads();
    if (pend >= 0) store_tile(pr, sh, int(threadIdx.x), row0, h, pend, chunk_tokens(T, pend));
    if (!producer && pr.s_out) {
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                pr.s_out[sbase + int64_t(16 * b + 4 * g + r) * kN + jcol] = S[b][r];
    }
}

// One token for every (row, head), one wave per head.  Lane (rg, cq) holds
// columns 4cq .. 4cq+3 of rows 4m + rg (m = 0 .. 15), so each of the wave's
// 16 loads and stores of the state covers 4 whole rows (1 KB).  The decay,
// key and receptance of the 64 key channels pass through LDS, ordered so that
// a lane's 16 rows are contiguous.
template <int DT, bool PER_TOKEN_Z>
__global__ __launch_bounds__(256) void mat_step_kernel(MatStepProblem pr) {
    __shared__ float tab[4][3][kN];  // per wave: d, k, r of key channel 4m + rg at rg * 16 + m
    const int wave = mat_wave();
    const int lane = mat_lane();
    const int64_t H = pr.H, C = H * kN;
    const int64_t head = int64_t(blockIdx.x) * 4 + wave;
    const bool live = head < pr.L * pr.S * H;
    const int64_t row = live ? head / H : 0;  // l * S + s
    const int64_t h = live ? head - row * H : 0;
    const int64_t layer = row / pr.S;
    const int64_t e0 = row * C + h * kN;
    if (live) {
        // lane = key channel
        const float z = PER_TOKEN_Z ? load_one<DT>(pr.z, e0 + lane)
                                    : static_cast<const float*>(pr.z)[layer * C + h * kN + lane];
        const int slot = (lane & 3) * 16 + (lane >> 2);
        tab[wave][0][slot] = decay_of(z);
        tab[wave][1][slot] = load_one<DT>(pr.k, e0 + lane);
        tab[wave][2][slot] = load_one<DT>(pr.r, e0 + lane);
    }
    __syncthreads();
    if (!live) return;
    const int rg = lane >> 4;
    const int cq = lane & 15;
    float vv[4];
    Quad<DT>::unpack(Quad<DT>::load(pr.v, e0 + 4 * cq), vv);
    const int64_t sb = head * int64_t(kN * kN) + int64_t(rg) * kN + 4 * cq;
    float4 st[16];
#pragma unroll
    for (int m = 0; m < 16; m++)
        st[m] = load_stream(reinterpret_cast<const float4*>(pr.s_in + sb + m * 4 * kN));
    float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
        const float4 d4 = *reinterpret_cast<const float4*>(&tab[wave][0][rg * 16 + 4 * q4]);
        const float4 k4 = *reinterpret_cast<const float4*>(&tab[wave][1][rg * 16 + 4 * q4]);
        const float4 r4 = *reinterpret_cast<const float4*>(&tab[wave][2][rg * 16 + 4 * q4]);
        const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
        const float kk[4] = {k4.x, k4.y, k4.z, k4.w};
        const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            float4& s4 = st[4 * q4 + j];   // row 4 (4 q4 + j) + rg
            s4.x = __builtin_fmaf(dd[j], s4.x, kk[j] * vv[0]);
            s4.y = __builtin_fmaf(dd[j], s4.y, kk[j] * vv[1]);
            s4.z = __builtin_fmaf(dd[j], s4.z, kk[j] * vv[2]);
            s4.w = __builtin_fmaf(dd[j], s4.w, kk[j] * vv[3]);
            y[0] = __builtin_fmaf(rr[j], s4.x, y[0]);
            y[1] = __builtin_fmaf(rr[j], s4.y, y[1]);
            y[2] = __builtin_fmaf(rr[j], s4.z, y[2]);
            y[3] = __builtin_fmaf(rr[j], s4.w, y[3]);
        }
    }
#pragma unroll
    for (int m = 0; m < 16; m++) *reinterpret_cast<float4*>(pr.s_out + sb + m * 4 * kN) = st[m];
    // the four row groups hold partial sums over disjoint rows
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const float y01 = y[c] + __shfl_xor(y[c], 16);
        y[c] = y01 + __shfl_xor(y01, 32);
    }
    if (rg == 0) Quad<DT>::store(pr.y, e0 + 4 * cq, y);
}

}  // namespace

hipError_t launch_mat_forward(const MatProblem& pr, hipStream_t stream) {
    const dim3 grid(unsigned(pr.B * pr.H)), block(512);
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
