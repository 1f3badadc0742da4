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
// Forward (training / prefill form): one workgroup of 8 waves per (batch row,
// head).  Consumer wave w (waves 0..3) owns value columns [16w, 16w + 16) of
// the state, which stays in fp32 registers in the accumulator layout of a
// 16x16 MFMA tile (lane l holds rows 4(l/16) .. 4(l/16)+3 of column l%16 of
// each of the four 16-row blocks); waves 4..7 prepare the chunks' operands.
// The tokens are taken in chunks of 16.  With D_t[i] the product of the decays
// d[i] of the chunk's tokens up to and including t, the recurrence unrolls
// over a chunk into
//
//   y_t = (r_t D_t)^T S_0 + sum_{s<=t} [sum_i r_t[i] D_t[i] k_s[i] / D_s[i]] v_s
//   S_16 = diag(D_15) S_0 + sum_s (k_s D_15 / D_s) v_s^T
//
// and every sum over i or s is a dense product on the matrix cores (bf16
// operands, fp32 accumulation): the read-out of the carried state, the
// chunk's score matrix, its application to the values, and the state update.
// The factor 1/D_s is bounded by the chunk's total decay; a chunk in which
// some channel decays by more than e^{-80} is run token by token instead, in
// fp32.  fp32 storage takes the token-by-token form throughout (its own
// kernel).
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

// The operand tiles of one chunk (chunked form) and its y tile.
struct ChunkOps {
    uint16_t rq[kCT][kRowPad];    // r_t[i] D_t[i]
    uint16_t kq[kCT][kRowPad];    // k_s[i] / D_s[i]
    uint16_t kdt[kN][kColPad];    // k_s[i] D_15[i] / D_s[i], [i][s]
    uint16_t vt[kN][kColPad];     // v_s[j], [j][s]
    float el[kN];                 // D_15[i]
    uint16_t yt[kCT][kRowPad];    // y of the chunk, written out afterwards
};

// The token-by-token kernel's fp32 inputs of a chunk, double-buffered by
// chunk parity; rows padded so that a wave's 16-byte writes spread over the
// banks.
struct TokShared {
    float rf[2][kCT][kN + 4], kf[2][kCT][kN + 4], df[2][kCT][kN + 4], vf[2][kCT][kN + 4];
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

__device__ __forceinline__ int chunk_tokens(int64_t T, int64_t ch) {
    const int64_t left = T - ch * kCT;  // <= 0 past the last chunk
    return left < kCT ? (left > 0 ? int(left) : 0) : kCT;
}

// Producer of the token-by-token kernel: the fp32 inputs of chunk ch into LDS
// buffer ch & 1.  Thread (tt, i0) handles token tt of the chunk and channels
// i0 .. i0+3.  Chunks past the last one are all padding (no decay, zero keys).
template <int DT, bool PER_TOKEN_Z>
__device__ __forceinline__ void stage_chunk(TokShared& sh, int tt, int i0, const ChunkIn<DT>& cur,
                                            const float (&dc)[4], int64_t T, int64_t ch) {
    using Q = Quad<DT>;
    const int buf = int(ch & 1);
    const bool live = tt < chunk_tokens(T, ch);
    float rv[4], kv[4], vv[4], dcy[4];
    Q::unpack(keep_if(live, cur.v), vv);
    Q::unpack(keep_if(live, cur.r), rv);
    Q::unpack(keep_if(live, cur.k), kv);
    if constexpr (PER_TOKEN_Z) {
        float zv[4];
        Q::unpack(pad_z(live, cur.z), zv);
#pragma unroll
        for (int c = 0; c < 4; c++) dcy[c] = decay_of(zv[c]);
    } else {
#pragma unroll
        for (int c = 0; c < 4; c++) dcy[c] = live ? dc[c] : 1.0f;
    }
    *reinterpret_cast<float4*>(&sh.rf[buf][tt][i0]) = make_float4(rv[0], rv[1], rv[2], rv[3]);
    *reinterpret_cast<float4*>(&sh.kf[buf][tt][i0]) = make_float4(kv[0], kv[1], kv[2], kv[3]);
    *reinterpret_cast<float4*>(&sh.df[buf][tt][i0]) = make_float4(dcy[0], dcy[1], dcy[2], dcy[3]);
    *reinterpret_cast<float4*>(&sh.vf[buf][tt][i0]) = make_float4(vv[0], vv[1], vv[2], vv[3]);
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

// The chunked form's operands of one consumer lane: rows 16b + 4g .. +3 of
// its token nn (rq, kq), key channels 16b + nn over tokens 4g .. +3 (kd), and
// value column jcol over the same tokens (v).
struct FastOps {
    short4_t rqB[4], kqA[4], kdA[4], vA;
};

__device__ __forceinline__ void read_ops(const ChunkOps& op, int g, int nn, int jcol, FastOps& f) {
#pragma unroll
    for (int b = 0; b < 4; b++) {
        f.rqB[b] = lds4(&op.rq[nn][16 * b + 4 * g]);
        f.kqA[b] = lds4(&op.kq[nn][16 * b + 4 * g]);
        f.kdA[b] = lds4(&op.kdt[16 * b + nn][4 * g]);
    }
    f.vA = lds4(&op.vt[jcol][4 * g]);
}

// One chunk on the matrix cores against the state S (accumulator layout:
// S[b][r] = S[16b + 4g + r][jcol]); y of the wave's 16 value columns goes to
// the tile op.yt.
__device__ __forceinline__ void consume_fast(ChunkOps& op, const FastOps& f, int wave, int g, int nn,
                                             float (&S)[4][4]) {
    float4_t yacc = {0.f, 0.f, 0.f, 0.f};
    float4_t aacc = {0.f, 0.f, 0.f, 0.f};
    // the contraction over the 64 key channels as two 16x16x32 products:
    // lane group g supplies rows 16b + 4g .. +3 of blocks b = 2m, 2m+1 (its
    // own state registers), and the same channels of rq and kq
#pragma unroll
    for (int m = 0; m < 2; m++) {
        const short4_t s0 = pack4(S[2 * m][0], S[2 * m][1], S[2 * m][2], S[2 * m][3]);
        const short4_t s1 = pack4(S[2 * m + 1][0], S[2 * m + 1][1], S[2 * m + 1][2], S[2 * m + 1][3]);
        yacc = mfma32(s0, s1, f.rqB[2 * m], f.rqB[2 * m + 1], yacc);
        aacc = mfma32(f.kqA[2 * m], f.kqA[2 * m + 1], f.rqB[2 * m], f.rqB[2 * m + 1], aacc);
    }
    // aacc[r] = score of key token s = 4g + r for query token nn; causal mask s <= t
    float am[4];
#pragma unroll
    for (int r = 0; r < 4; r++) am[r] = (4 * g + r <= nn) ? aacc[r] : 0.0f;
    yacc = mfma16(f.vA, pack4(am[0], am[1], am[2], am[3]), yacc);
    // yacc[r] = y[token nn][column 16 wave + 4g + r], into the tile: a
    // wave's direct stores would write 32 bytes of each of 16 rows
    *reinterpret_cast<uint2*>(&op.yt[nn][16 * wave + 4 * g]) =
        make_uint2(bf16_word(yacc[0], yacc[1]), bf16_word(yacc[2], yacc[3]));
    // S <- diag(D_15) S + Kd^T V: the product does not wait for D_15
    float4_t upd[4];
#pragma unroll
    for (int b = 0; b < 4; b++) upd[b] = mfma16(f.kdA[b], f.vA, float4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const float4 e4 = *reinterpret_cast<const float4*>(&op.el[16 * b + 4 * g]);
        S[b][0] = __builtin_fmaf(S[b][0], e4.x, upd[b][0]);
        S[b][1] = __builtin_fmaf(S[b][1], e4.y, upd[b][1]);
        S[b][2] = __builtin_fmaf(S[b][2], e4.z, upd[b][2]);
        S[b][3] = __builtin_fmaf(S[b][3], e4.w, upd[b][3]);
    }
}

// One chunk token by token in fp32, y of the wave's 16 value columns written
// to global memory at once.  FROM_LDS: the inputs are the fp32 arrays of
// buffer buf (fp32 storage); otherwise they are read from global memory (the
// rare chunk of the chunked kernel whose decay is too steep for it).
template <int DT, bool PER_TOKEN_Z, bool FROM_LDS>
__device__ __forceinline__ void consume_tokens(const MatProblem& pr, const TokShared* sh, int buf, int g,
                                               int jcol, int64_t row0, int64_t h, int64_t ch,
                                               float (&S)[4][4]) {
    const int64_t C = pr.H * kN;
    const int64_t t0 = ch * kCT;
    const int n = chunk_tokens(pr.T, ch);
    for (int t = 0; t < n; t++) {
        const int64_t e = (row0 + t0 + t) * C + h * kN;
        float vj;
        if constexpr (FROM_LDS) vj = sh->vf[buf][t][jcol];
        else vj = load_one<DT>(pr.v, e + jcol);
        float yp = 0.0f;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            float dd[4], kk[4], rr[4];
            if constexpr (FROM_LDS) {
                const float4 d4 = *reinterpret_cast<const float4*>(&sh->df[buf][t][16 * b + 4 * g]);
                const float4 k4 = *reinterpret_cast<const float4*>(&sh->kf[buf][t][16 * b + 4 * g]);
                const float4 r4 = *reinterpret_cast<const float4*>(&sh->rf[buf][t][16 * b + 4 * g]);
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
}

// Chunks in flight per producer thread: the inputs of the next kPrefetch
// chunks are loaded into registers while the current one is processed.
constexpr int kPrefetch = 4;

// Token-by-token form (fp32 storage, or on request): one workgroup of 8 waves
// per (batch row, head).  Waves 4..7 stage the fp32 inputs of chunk c+1 in LDS
// while waves 0..3 run chunk c token by token against their 16 value columns
// of the state; one barrier per chunk hands the double-buffered LDS over.
// Workgroup -> (batch row, head) task.  Heads 2j and 2j + 1 of a row (the
// two 128-byte halves of a 256-byte piece of every row) go to workgroups j
// and j + n/2: the dispatcher deals workgroups to the XCDs in turn and fills
// the CUs in the same order in its second round, so the pair runs on one XCD
// (one CU, in practice) and the halves of each row reach memory together.
// A probe of this kernel's access pattern alone (4 reads and 1 write in
// 128-byte pieces of the bf16 [16, 4096, 2048] rows) takes 288 us with the
// plain order and 250 us paired, as fast as 256-byte pieces.  Any bijection
// is correct; an odd count keeps the plain order.
__device__ __forceinline__ int64_t paired_task(int64_t bid, int64_t n) {
    if (n & 1) return bid;
    const int64_t half = n / 2;
    return bid < half ? 2 * bid : 2 * (bid - half) + 1;
}

template <int DT, bool PER_TOKEN_Z>
__global__ __launch_bounds__(512, 4) void mat_forward_tokens_kernel(MatProblem pr) {
    __shared__ TokShared sh;
    const int wave = mat_wave();
    const int lane = mat_lane();
    const bool producer = wave >= 4;
    const int64_t T = pr.T, C = pr.H * kN;
    const int64_t task = paired_task(blockIdx.x, gridDim.x);
    const int64_t bb = task / pr.H;
    const int64_t h = task - bb * pr.H;
    const int64_t row0 = bb * T;
    const int64_t nch = (T + kCT - 1) / kCT;
    // producer role: token tt of a chunk, channels i0 .. i0+3
    const int tt = lane & 15;
    const int i0 = 4 * (4 * (wave & 3) + (lane >> 4));
    // consumer role: lane group g, column jcol of the state
    const int g = lane >> 4;
    const int jcol = 16 * (wave & 3) + (lane & 15);

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
    // the state and decay loads complete here (s_waitcnt vmcnt(0) as an
    // instruction the compiler's wait insertion sees), so that the waits inside
    // the chunk loop only count the prefetch ring's loads
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // element offset of token tt of chunk ch (ch >= 0), clamped to the last
    // token; only called when T >= 1
    const int64_t e0 = row0 * C + h * kN + i0;
    auto elem = [&](int64_t ch) {
        const int64_t t = ch * kCT + tt;
        return e0 + (t < T ? t : T - 1) * C;
    };
    // The producers keep a ring of kPrefetch chunks in registers: slot p is
    // staged, then reloaded in place with the chunk kPrefetch ahead.  Loads
    // are unconditional (chunks past the last one load the last token; their
    // values are masked as padding).  In the interval of chunk q the producers
    // stage q while the consumers run q - 1.  The two roles run separate loops
    // (so that neither holds the other's registers) with the same number of
    // barriers; nothing happens for T = 0.
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
                    if (q0 >= 0) stage_chunk<DT, PER_TOKEN_Z>(sh, tt, i0, ring[p], dc, T, q);
                    load_chunk<DT, PER_TOKEN_Z>(ring[p], pr, elem(q + kPrefetch));
                    if (q0 >= 0) __syncthreads();
                }
            }
        } else {
            for (int64_t q0 = 0; q0 <= nch; q0 += kPrefetch) {
#pragma unroll
                for (int p = 0; p < kPrefetch; p++) {
                    const int64_t q = q0 + p;
                    if (q >= 1 && q <= nch)
                        consume_tokens<DT, PER_TOKEN_Z, true>(pr, &sh, int((q - 1) & 1), g, jcol, row0, h, q - 1, S);
                    __syncthreads();
                }
            }
        }
    }
    if (!producer && pr.s_out) {
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                pr.s_out[sbase + int64_t(16 * b + 4 * g + r) * kN + jcol] = S[b][r];
    }
}

// ---------------------------------------------------------------------------
// Chunked form with a ring of operand tiles (bf16 storage).
//
// One workgroup of 8 waves per (batch row, head), as in the token-by-token
// kernel, but the two roles are not in lockstep: producer wave p (waves
// 4..7) prepares chunks p, p + 4, p + 8, ... on its own, each into ring slot
// (chunk mod 4), while the four consumer waves take the chunks in order.  Per slot, `ready` names the chunk
// whose operands are in it and `done` counts the consumer waves' completions
// of its chunks (4 per chunk), so chunk q may be written once it reaches
// 4 (q / 4).  The producer that takes a slot over first writes the previous
// chunk's y tile out of it, which keeps the stores off the consumers' path.
// The flags live in LDS; waits poll them.
//
// A producer lane (g, n) = (lane / 16, lane % 16) holds tokens 4g .. 4g+3 of
// its chunk for channels 4n .. 4n+3, so each of its loads covers four whole
// 128-byte rows of the head: the decay products run along its own four tokens,
// then across the four lane groups.
// ---------------------------------------------------------------------------

constexpr int kProducers = 4;                   // producer waves (chunk q to wave q mod 4)
constexpr int kSlots = 6;                       // ring slots (chunk q to slot q mod 6)
constexpr uint64_t kRingSpinTicks = 20000000;   // 200 ms of the 100 MHz real-time counter
constexpr int kProducerSleep = 4;               // producers wait for a free slot at a slower poll

// Count of ring workgroups whose bounded waits gave up, on this device, since
// the library was loaded (read by wkv_bounded_wait_failures()).
__device__ unsigned int g_ring_wait_failures;

struct MatRing {
    ChunkOps slot[kSlots];
    int ready[kSlots];   // chunk whose operands the slot holds (-1: none yet)
    int done[kSlots];    // consumer waves' completions of the slot's chunks, in all
    int exact[kSlots];   // 1 when the slot's chunk must run token by token
    int gave_up;         // set once a wait timed out: no later wait blocks
};

// Wait until *f == want.  The wait is bounded, and once one wait of the
// workgroup has given up no other blocks: a slip in the hand-over ends the
// workgroup, which then writes NaN over its outputs and state and counts
// itself in g_ring_wait_failures (never expected; see the end of the kernel).
// SLEEP: the pause between polls (units of 64 cycles).
template <int SLEEP>
__device__ __forceinline__ void ring_wait(MatRing& sh, int* f, int want) {
    if (__hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == want) return;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (uint32_t i = 1;; i++) {
        __builtin_amdgcn_s_sleep(SLEEP);
        if (__hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == want) return;
        // the clock and the give-up flag are looked at every 16th poll
        if ((i & 15) == 0) {
            if (__hip_atomic_load(&sh.gave_up, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) return;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kRingSpinTicks) {
                __hip_atomic_store(&sh.gave_up, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                return;
            }
        }
    }
}

// The raw bf16 inputs of one chunk held by a producer lane: word pair j is
// token 4g + j, channels 4n .. 4n+3.
struct RawChunk {
    u32x2_t r[4], k[4], v[4], z[4];
};

// Buffer descriptor of chunk q of one array: its first row at channel h * 64.
// Rows past the sequence end read as zero (the descriptor's size stops at the
// last valid row's head channels); chunks past the last one read nothing.
__device__ __forceinline__ rsrc_t ring_rsrc(const void* base, int64_t row0, int64_t T, int64_t C,
                                            int64_t h, int64_t q, int64_t nch) {
    const bool in = q < nch;
    const int64_t t0 = in ? q * kCT : 0;
    const int64_t rows = in ? (T - t0 < kCT ? T - t0 : kCT) : 0;
    const int64_t row_bytes = C * 2;
    const int num = rows == kCT ? -1 : int(rows > 0 ? rows * row_bytes - h * kN * 2 : 0);
    const char* p = static_cast<const char*>(base) + ((row0 + t0) * C + h * kN) * 2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, num, 0x00020000);
}

// The loads of chunk q: voff[j] is the byte offset of the lane's word pair j
// (token 4g + j, channel 4n) from the chunk's first row.  The whole offset is
// in the vector operand, where the descriptor's size check applies to it.
template <bool PER_TOKEN_Z>
__device__ __forceinline__ void ring_load(RawChunk& x, const MatProblem& pr, int64_t row0, int64_t h,
                                          int64_t q, int64_t nch, const uint32_t (&voff)[4]) {
    const int64_t T = pr.T, C = pr.H * kN;
    const rsrc_t rr = ring_rsrc(pr.r, row0, T, C, h, q, nch);
    const rsrc_t kr = ring_rsrc(pr.k, row0, T, C, h, q, nch);
    const rsrc_t vr = ring_rsrc(pr.v, row0, T, C, h, q, nch);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        x.r[j] = __builtin_amdgcn_raw_buffer_load_b64(rr, voff[j], 0u, kStreamLoad);
        x.k[j] = __builtin_amdgcn_raw_buffer_load_b64(kr, voff[j], 0u, kStreamLoad);
        x.v[j] = __builtin_amdgcn_raw_buffer_load_b64(vr, voff[j], 0u, kStreamLoad);
    }
    if constexpr (PER_TOKEN_Z) {
        const rsrc_t zr = ring_rsrc(pr.z, row0, T, C, h, q, nch);
#pragma unroll
        for (int j = 0; j < 4; j++) x.z[j] = __builtin_amdgcn_raw_buffer_load_b64(zr, voff[j], 0u, kStreamLoad);
    }
}

__device__ __forceinline__ void unpack_bf16x4(u32x2_t w, float (&x)[4]) {
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
}

// Value of lane `src` of the wave.
__device__ __forceinline__ float lane_value(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// The y tile of chunk q, consumed from slot s, to global memory in whole
// 128-byte rows.  Nothing is written when `any` is false (no chunk) or the
// chunk ran token by token (y is out already): the stores then go through a
// zero-size descriptor, and rows past the sequence end past the descriptor's
// size, so that the four stores are issued on every path (a branch around
// them would make later waits for the loads wait for every store as well).
__device__ __forceinline__ void ring_store_tile(const MatProblem& pr, MatRing& sh, int s, int64_t q, bool any,
                                                int lane, int64_t row0, int64_t h) {
    const int64_t C = pr.H * kN, T = pr.T;
    const int g = lane >> 4, nn = lane & 15;
    const bool write = any && sh.exact[s] == 0;
    const int64_t t0 = any ? q * kCT : 0;
    const int64_t rows = T - t0 < kCT ? T - t0 : kCT;
    const uint32_t row_bytes = uint32_t(C * 2);
    const int num = !write ? 0 : (rows == kCT ? -1 : int(rows * int64_t(row_bytes) - h * kN * 2));
    char* p = static_cast<char*>(pr.y) + ((row0 + t0) * C + h * kN) * 2;
    const rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(p, (short)0, num, 0x00020000);
    const ChunkOps& op = sh.slot[s];
    u32x2_t yv[4];
#pragma unroll
    for (int i = 0; i < 4; i++) yv[i] = *reinterpret_cast<const u32x2_t*>(&op.yt[4 * i + g][4 * nn]);
#pragma unroll
    for (int i = 0; i < 4; i++)
        __builtin_amdgcn_raw_buffer_store_b64(yv[i], yr, uint32_t(4 * i + g) * row_bytes + uint32_t(8 * nn), 0u,
                                              kStreamStore);
}

// Producer: the operand tiles of chunk q from the lane's raw inputs into ring
// slot q mod kSlots, once the slot is free; then the slot is published.
template <bool PER_TOKEN_Z>
__device__ __forceinline__ void ring_produce(const MatProblem& pr, MatRing& sh, const RawChunk& x,
                                             const float (&dc)[4], int lane, int64_t row0, int64_t h,
                                             int64_t q) {
    const int64_t T = pr.T;
    const int g = lane >> 4, n = lane & 15;
    const int s = int(q % kSlots);
    // the slot is free once the consumers are done with its previous chunk,
    // kSlots back; that chunk's y tile goes out first (the chunks ahead leave
    // time for it)
    ring_wait<kProducerSleep>(sh, &sh.done[s], 4 * int(q / kSlots));
    ring_store_tile(pr, sh, s, q - kSlots, q >= kSlots, lane, row0, h);
    const int live = chunk_tokens(T, q);   // tokens of the chunk; 4g + j >= live is padding
    // decays d[j][c] of token 4g + j, channel 4n + c; padding tokens do not decay
    float d[4][4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        if constexpr (PER_TOKEN_Z) {
            float zv[4];
            unpack_bf16x4(x.z[j], zv);
#pragma unroll
            for (int c = 0; c < 4; c++) d[j][c] = decay_of(4 * g + j < live ? zv[c] : -__builtin_inff());
        } else {
#pragma unroll
            for (int c = 0; c < 4; c++) d[j][c] = 4 * g + j < live ? dc[c] : 1.0f;
        }
    }
    // D[j][c] = product of the chunk's decays up to token 4g + j: along the
    // lane's own tokens, then the products of the lane groups before it
    float D[4][4], DL[4];
    bool wide = false;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        D[0][c] = d[0][c];
#pragma unroll
        for (int j = 1; j < 4; j++) D[j][c] = D[j - 1][c] * d[j][c];
        // (the lane reads are taken by every lane: a read from a lane that
        // is switched off returns nothing useful)
        const float t = D[3][c];                                         // group g's product
        const float u1 = lane_value(t, lane - 16);
        const float t1 = g >= 1 ? t * u1 : t;                            // groups g-1 .. g
        const float u2 = lane_value(t1, lane - 32);
        const float t2 = g >= 2 ? t1 * u2 : t1;                          // groups 0 .. g
        const float before = lane_value(t2, lane - 16);                  // groups 0 .. g-1
        const float e = g >= 1 ? before : 1.0f;
        DL[c] = lane_value(t2, 48 + n);                                  // the whole chunk
#pragma unroll
        for (int j = 0; j < 4; j++) D[j][c] *= e;
        wide = wide || !(DL[c] >= kMinChunkDecay);
    }
    // rq = r D, kq = k / D, kd = k D_15 / D in bf16
    uint32_t rq[4][2], kq[4][2], kd[4][2];   // [token j][channel pair]; kd: [channel c][token pair]
    float kdv[4][4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        float rv[4], kv[4], q4[4], r4[4];
        unpack_bf16x4(x.r[j], rv);
        unpack_bf16x4(x.k[j], kv);
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const float inv = __builtin_amdgcn_rcpf(D[j][c]);
            r4[c] = rv[c] * D[j][c];
            q4[c] = kv[c] * inv;
            kdv[j][c] = q4[c] * DL[c];
        }
        rq[j][0] = bf16_word(r4[0], r4[1]);
        rq[j][1] = bf16_word(r4[2], r4[3]);
        kq[j][0] = bf16_word(q4[0], q4[1]);
        kq[j][1] = bf16_word(q4[2], q4[3]);
    }
#pragma unroll
    for (int c = 0; c < 4; c++) {
        kd[c][0] = bf16_word(kdv[0][c], kdv[1][c]);
        kd[c][1] = bf16_word(kdv[2][c], kdv[3][c]);
    }
    // v as stored, regrouped from [token][channel] to [channel][token] words:
    // channel c of tokens 0, 1 (then 2, 3) = 16-bit half c of words j, j + 1
    uint32_t vt[4][2];
#pragma unroll
    for (int c = 0; c < 4; c++) {
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const uint32_t lo = (c < 2) ? x.v[2 * p].x : x.v[2 * p].y;
            const uint32_t hi = (c < 2) ? x.v[2 * p + 1].x : x.v[2 * p + 1].y;
            // selector: bytes of hi are 4..7, of lo 0..3; low half of a word is bytes 0, 1
            vt[c][p] = (c & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u) : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
    }
    const bool exact = __builtin_amdgcn_ballot_w64(wide) != 0;

    ChunkOps& op = sh.slot[s];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        *reinterpret_cast<uint2*>(&op.rq[4 * g + j][4 * n]) = make_uint2(rq[j][0], rq[j][1]);
        *reinterpret_cast<uint2*>(&op.kq[4 * g + j][4 * n]) = make_uint2(kq[j][0], kq[j][1]);
    }
#pragma unroll
    for (int c = 0; c < 4; c++) {
        *reinterpret_cast<uint2*>(&op.kdt[4 * n + c][4 * g]) = make_uint2(kd[c][0], kd[c][1]);
        *reinterpret_cast<uint2*>(&op.vt[4 * n + c][4 * g]) = make_uint2(vt[c][0], vt[c][1]);
    }
    if (g == 0) *reinterpret_cast<float4*>(&op.el[4 * n]) = make_float4(DL[0], DL[1], DL[2], DL[3]);
    if (lane == 0) {
        sh.exact[s] = exact ? 1 : 0;
        __hip_atomic_store(&sh.ready[s], int(q), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

// A consumer wave is done with the chunk in slot s (its operand reads and its
// part of the y tile complete before the count).
__device__ __forceinline__ void ring_finish(MatRing& sh, int s, int lane) {
    if (lane == 0) __hip_atomic_fetch_add(&sh.done[s], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <bool PER_TOKEN_Z>
__global__ __launch_bounds__(512, 4) void mat_forward_ring_kernel(MatProblem pr) {
    __shared__ MatRing sh;
    const int wave = mat_wave();
    const int lane = mat_lane();
    const bool producer = wave >= 4;
    const int64_t T = pr.T, C = pr.H * kN;
    const int64_t task = paired_task(blockIdx.x, gridDim.x);
    const int64_t bb = task / pr.H;
    const int64_t h = task - bb * pr.H;
    const int64_t row0 = bb * T;
    const int64_t nch = (T + kCT - 1) / kCT;
    const int g = lane >> 4;
    const int nn = lane & 15;

    float S[4][4];
    const int64_t sbase = (bb * pr.H + h) * int64_t(kN * kN);
    const int jcol = 16 * (wave & 3) + nn;
    if (!producer) {
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                S[b][r] = pr.s_in ? pr.s_in[sbase + int64_t(16 * b + 4 * g + r) * kN + jcol] : 0.0f;
    }
    // per-channel decay (Eagle) of the producer lane's channels 4 nn .. 4 nn + 3
    float dc[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (!PER_TOKEN_Z) {
        if (producer) {
#pragma unroll
            for (int c = 0; c < 4; c++) dc[c] = decay_of(static_cast<const float*>(pr.z)[h * kN + 4 * nn + c]);
        }
    }
    if (threadIdx.x == 0) sh.gave_up = 0;
    if (threadIdx.x < kSlots) {
        sh.ready[threadIdx.x] = -1;
        sh.done[threadIdx.x] = 0;
        sh.exact[threadIdx.x] = 0;
    }
    // the state and decay loads complete here (s_waitcnt vmcnt(0) as an
    // instruction the compiler's wait insertion sees), so that the waits in
    // the loops only count the loads of the chunks in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    if (producer) {
        const int p = wave - 4;
        const uint32_t row_bytes = uint32_t(C * 2);
        uint32_t voff[4];
#pragma unroll
        for (int j = 0; j < 4; j++) voff[j] = uint32_t(4 * g + j) * row_bytes + uint32_t(8 * nn);
        // two register sets: the wave's next chunk loads while this one is prepared
        RawChunk xa, xb;
        ring_load<PER_TOKEN_Z>(xa, pr, row0, h, p, nch, voff);
        for (int64_t q = p; q < nch; q += 2 * kProducers) {
            ring_load<PER_TOKEN_Z>(xb, pr, row0, h, q + kProducers, nch, voff);
            ring_produce<PER_TOKEN_Z>(pr, sh, xa, dc, lane, row0, h, q);
            if (q + kProducers >= nch) break;
            ring_load<PER_TOKEN_Z>(xa, pr, row0, h, q + 2 * kProducers, nch, voff);
            ring_produce<PER_TOKEN_Z>(pr, sh, xb, dc, lane, row0, h, q + kProducers);
        }
        // each slot's last chunk (slot s by producer s mod 4): its y tile once
        // the consumers are done with it
        for (int s = p; s < kSlots; s += kProducers) {
            if (s < nch) {
                const int64_t last = s + (nch - 1 - s) / kSlots * kSlots;
                ring_wait<kProducerSleep>(sh, &sh.done[s], 4 * int(last / kSlots + 1));
                ring_store_tile(pr, sh, s, last, true, lane, row0, h);
            }
        }
    } else {
        // chunks in pairs: the two chunks' products are independent but for
        // the state, so their latencies overlap
        for (int64_t q = 0; q < nch; q += 2) {
            const int64_t q1 = q + 1;
            const bool two = q1 < nch;
            const int s0 = int(q % kSlots), s1 = int(q1 % kSlots);
            ring_wait<1>(sh, &sh.ready[s0], int(q));
            if (two) ring_wait<1>(sh, &sh.ready[s1], int(q1));
            const bool fast0 = sh.exact[s0] == 0;
            const bool fast1 = two && sh.exact[s1] == 0;
            if (fast0 && fast1) {
                FastOps f0, f1;
                read_ops(sh.slot[s0], g, nn, jcol, f0);
                read_ops(sh.slot[s1], g, nn, jcol, f1);
                consume_fast(sh.slot[s0], f0, wave, g, nn, S);
                consume_fast(sh.slot[s1], f1, wave, g, nn, S);
            } else {
                // one chunk at a time (the last one, or a token-by-token one)
                for (int i = 0; i < (two ? 2 : 1); i++) {
                    const int si = i == 0 ? s0 : s1;
                    if (i == 0 ? fast0 : fast1) {
                        FastOps f;
                        read_ops(sh.slot[si], g, nn, jcol, f);
                        consume_fast(sh.slot[si], f, wave, g, nn, S);
                    } else {
                        consume_tokens<kBF16, PER_TOKEN_Z, false>(pr, nullptr, 0, g, jcol, row0, h, q + i, S);
                    }
                }
            }
            ring_finish(sh, s0, lane);
            if (two) ring_finish(sh, s1, lane);
        }
        if (pr.s_out) {
#pragma unroll
            for (int b = 0; b < 4; b++)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    pr.s_out[sbase + int64_t(16 * b + 4 * g + r) * kN + jcol] = S[b][r];
        }
    }
    // every wave gets here (all waits are bounded).  A wait that gave up
    // leaves the head's results unusable: they are overwritten with NaN, so
    // no check of finite outputs can miss it, and the miss is counted.
    __syncthreads();
    if (__hip_atomic_load(&sh.gave_up, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) {
        uint16_t* y = static_cast<uint16_t*>(pr.y);
        for (int64_t t = threadIdx.x / kN; t < T; t += blockDim.x / kN)
            y[(row0 + t) * C + h * kN + threadIdx.x % kN] = 0x7FC0u;   // bf16 NaN
        if (pr.s_out)
            for (int e = threadIdx.x; e < kN * kN; e += blockDim.x) pr.s_out[sbase + e] = __builtin_nanf("");
        if (threadIdx.x == 0) atomicAdd(&g_ring_wait_failures, 1u);
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
    // non-temporal stores of the state (830 -> 808 us on the decode workload),
    // through plain pointers like its loads: stored through a buffer
    // descriptor (either cache policy) while loaded through plain pointers,
    // the in-place state came out nondeterministic at the decode workload's
    // size (two eager runs from one state differing in a few heads), where
    // loads and stores both through the descriptor were deterministic; the
    // cause inside that mix was not found (tests/test_gpu_graph.py checks the
    // full size)
#pragma unroll
    for (int m = 0; m < 16; m++) store_stream(reinterpret_cast<float4*>(pr.s_out + sb + m * 4 * kN), st[m]);
    // the four row groups hold partial sums over disjoint rows
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const float y01 = y[c] + __shfl_xor(y[c], 16);
        y[c] = y01 + __shfl_xor(y01, 32);
    }
    if (rg == 0) Quad<DT>::store(pr.y, e0 + 4 * cq, y);
}

}  // namespace

hipError_t read_ring_wait_failures(uint64_t* count) {
    unsigned int n = 0;
    const hipError_t e = hipMemcpyFromSymbol(&n, HIP_SYMBOL(g_ring_wait_failures), sizeof(n), 0,
                                             hipMemcpyDeviceToHost);
    *count = n;
    return e;
}

hipError_t launch_mat_forward(const MatProblem& pr, hipStream_t stream) {
    const dim3 grid(unsigned(pr.B * pr.H)), block(512);
    // the ring kernel's byte offsets within a chunk are 32-bit
    const bool tokens = pr.dtype == kF32 || pr.path == 1 || pr.H * kN * 2 * kCT >= (int64_t(1) << 31);
#define WKV_MAT_TOK(DT, PT) hipLaunchKernelGGL((mat_forward_tokens_kernel<DT, PT>), grid, block, 0, stream, pr)
#define WKV_MAT_RING(PT) hipLaunchKernelGGL((mat_forward_ring_kernel<PT>), grid, block, 0, stream, pr)
    if (pr.dtype == kF32) {
        if (pr.z_per_token) WKV_MAT_TOK(kF32, true);
        else WKV_MAT_TOK(kF32, false);
    } else if (tokens) {
        if (pr.z_per_token) WKV_MAT_TOK(kBF16, true);
        else WKV_MAT_TOK(kBF16, false);
    } else {
        if (pr.z_per_token) WKV_MAT_RING(true);
        else WKV_MAT_RING(false);
    }
#undef WKV_MAT_TOK
#undef WKV_MAT_RING
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
