// Device-side building blocks of the WKV kernels (gfx950, wave64).
//
// The operator ([tm-math] = aicassindra.com tm_rwkv_math, "The WKV operator:
// attention with a fixed decay"; "Numerical stability: carry the exponent"):
// per channel, state (a, b, p) with true accumulators e^p a, e^p b; per token
//
//   read-out  y  = (e^{p} a + e^{u+k} v) / (e^{p} b + e^{u+k})    (history + bonus)
//   fold-in   p' = max(p - w, k)
//             a' = e^{p-w-p'} a + e^{k-p'} v,   b' = e^{p-w-p'} b + e^{k-p'}
//
// How it is evaluated here (fp32 throughout; every exp argument is <= 0):
//
// 1. Exponents stay in natural-log units; a weight e^{x} is v_exp_f32 of
//    x log2 e, and the multiply by log2 e is applied to differences of
//    exponents (small where it matters), never to the exponents themselves.
//
// 2. One exponential per token.  With d the exponent of the decayed history
//    minus that of the new token, exactly one of the two weights is e^0 = 1
//    and the other is e = e^{-|d|}:
//      d >= 0:  alpha = 1, beta = e   (the history keeps the maximum)
//      d <  0:  alpha = e, beta = 1   (the new token becomes the maximum)
//
// 3. The read-out reuses the fold-in weights.  Multiplying numerator and
//    denominator of the read-out by e^{-w-p'} gives
//      y = (alpha a + beta c v) / (alpha b + beta c),   c = e^{u-w}
//    -- the same ratio with one per-channel constant and no second
//    exponential.  It is used when |u - w| <= 44 (c within [2^-64, 2^64]);
//    other channels take the read-out as written, with its own single
//    exponential.
//
// 4. No rounding accumulates in the running maximum.  Subtracting w from p at
//    every token would round at every token, and over many tokens the error
//    in p (which sets the weight of the whole history against each new token)
//    grows linearly.  Instead, inside a block of tokens the maximum is held
//    as an anchor `kas` in the frame of the block start: before token i of
//    the block p = kas - i w, and the new key enters the frame as
//    r = k + (i+1) w (one fma).  Then d = kas - r and the new anchor is
//    max(kas, r); nothing is subtracted token by token.  Between blocks the
//    state carries the anchor A and an exact token count m (p = A - m w),
//    so each exponent is formed with a couple of roundings however long the
//    sequence is.
//
// 5. exp is v_exp_f32 (2^x); the division is v_rcp_f32 and a multiply.  Both
//    are within about 1 ulp.
//
// 6. The empty history has exponent kEmptyP (a large finite negative), so
//    differences of two empty exponents are 0 rather than NaN.
//
// 7. Chunks.  Over a span of n tokens a state X becomes e^{-n w} X + G
//    ([tm-math] "Why it collapses into a recurrence": every older term gains
//    one factor e^{-w} per token), where G is the span's own state started
//    from the empty history.  In (a, b, A, m) form that is combine() below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kEmptyP = -1.0e38f;      // the empty history's exponent
constexpr float kEmptyIn = -1.0e30f;     // state inputs at or below this are empty
constexpr float kFusedMaxAbsUW = 44.0f;  // |u - w| bound for the fused read-out
constexpr float kNarrowMaxAbsUW = 13.8f; // |u - w| bound (c within [2^-20, 2^20]) for frame weights

enum : int { kF32 = 0, kBF16 = 1 };

// e^{-|d|}
__device__ __forceinline__ float exp_neg_abs(float d) {
    return __builtin_amdgcn_exp2f(-__builtin_fabsf(d * kLog2e));
}
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// A state kept between kernels in two numbers per channel: r = a / b, the
// history's weighted mean of v, and q = p + ln b, the log of its total weight
// (so a e^p = r e^q and b e^p = e^q: the same state, one rounding each).  The
// empty history is (0, kEmptyP).
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ void to_saved(float a, float b, float p, float& r, float& q) {
    const bool empty = !(b > 0.0f);
    r = empty ? 0.0f : a * fast_rcp(b);
    q = empty ? kEmptyP : __builtin_fmaf(__builtin_amdgcn_logf(b), kLn2, p);
}
__device__ __forceinline__ void from_saved(float r, float q, float& a, float& b, float& p) {
    const bool empty = q <= kEmptyIn;
    a = r;
    b = empty ? 0.0f : 1.0f;
    p = empty ? kEmptyP : q;
}

// 1 + e^{-r}: the receptance gate sigmoid(r) = 1 / (1 + e^{-r}) is applied as
// a factor of the read-out's denominator.
__device__ __forceinline__ float gate_den(float r) { return 1.0f + __builtin_amdgcn_exp2f(-r * kLog2e); }

// max(a, b) of two numbers that are never NaN, as one v_max_f32: the
// compiler's fmaxf first quiets every operand it cannot prove canonical,
// which costs two more instructions per call in the token loop.
__device__ __forceinline__ float max_num(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ float max3_num(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float min_num(float a, float b) {
    float r;
    asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Per-channel constants of the forward kernels.
struct Chan {
    float w;     // decay rate
    float wmu;   // w - u
    float c;     // e^{u-w}
    bool fused;  // fused read-out allowed
    bool narrow; // c within [2^-20, 2^20]: the frame-weight output pass applies
};

__device__ __forceinline__ Chan make_chan(float w, float u) {
    Chan ch;
    ch.w = w;
    ch.wmu = w - u;
    ch.fused = __builtin_fabsf(ch.wmu) <= kFusedMaxAbsUW;
    ch.narrow = __builtin_fabsf(ch.wmu) <= kNarrowMaxAbsUW;
    ch.c = __builtin_amdgcn_exp2f(ch.fused ? -ch.wmu * kLog2e : 0.0f);
    return ch;
}

// One token inside a frame (see 4.).  ip1 = i + 1 for token i of the frame.
// Updates a, b and the anchor kas; returns y.  `keep` is false when the new
// token became the maximum.
//
// GATED: the output is sigmoid(r) * y (the receptance gate, [tm-math]
// "Receptance: the gate on the way out"), passed in as gd = 1 + e^{-r}: the
// read-out's denominator is multiplied by gd, so the gate costs no second
// reciprocal.  gd = inf (r very negative) gives 0, the gate's limit.
template <bool FUSED_ONLY, bool GATED = false>
__device__ __forceinline__ float frame_token(float& a, float& b, float& kas, float k, float v,
                                             const Chan& ch, float ip1, bool& keep_out,
                                             float gd = 1.0f) {
    const float r = __builtin_fmaf(ip1, ch.w, k);  // new key in the block frame
    const float d = kas - r;                       // decayed history minus new token
    const float e = exp_neg_abs(d);
    const bool keep = d >= 0.0f;
    const float alpha = keep ? 1.0f : e;
    const float beta = keep ? e : 1.0f;
    const float t1 = alpha * a;
    float y;
    if (FUSED_ONLY || ch.fused) {
        const float delta = beta * ch.c;
        const float den = __builtin_fmaf(alpha, b, delta);
        y = __builtin_fmaf(delta, v, t1) * fast_rcp(GATED ? den * gd : den);
    } else {
        // read-out as written: history exponent p = kas - i w against u + k
        const float dr = d + ch.wmu;
        const float er = exp_neg_abs(dr);
        const bool kr = dr >= 0.0f;
        const float ar = kr ? 1.0f : er;
        const float br = kr ? er : 1.0f;
        const float den = __builtin_fmaf(ar, b, br);
        y = __builtin_fmaf(br, v, ar * a) * fast_rcp(GATED ? den * gd : den);
    }
    a = __builtin_fmaf(beta, v, t1);
    b = __builtin_fmaf(alpha, b, beta);
    kas = max_num(kas, r);
    keep_out = keep;
    return y;
}

// X <- X (+) G: G is the state of the n tokens that follow X, started from
// the empty history; both in anchor form (exponent = A - m w).
__device__ __forceinline__ void combine(float& xa, float& xb, float& xA, float& xm, float ga,
                                        float gb, float gA, float gm, float n, float w) {
    const float xm2 = xm + n;
    const float px = __builtin_fmaf(-xm2, w, xA);
    const float pg = __builtin_fmaf(-gm, w, gA);
    const float d = px - pg;
    const float e = exp_neg_abs(d);
    const bool keep = d >= 0.0f;
    const float alpha = keep ? 1.0f : e;
    const float beta = keep ? e : 1.0f;
    xa = __builtin_fmaf(beta, ga, alpha * xa);
    xb = __builtin_fmaf(beta, gb, alpha * xb);
    xA = keep ? xA : gA;
    xm = keep ? xm2 : gm;
}

// Decode step.  The state is stored after every token, so whatever it holds
// is rounded once per token.  Storing p' = fl(p - w) would round the
// exponent of the whole history at every token, and with w fixed that
// rounding goes the same way token after token: the history's weight drifts
// against every new key (1e-4 after a few hundred tokens behind a key near
// +40).  Instead the exponent is an anchor that stays where it is while no
// new key exceeds it, and the decay is applied to the sums: a, b are
// multiplied by D = e^{-w} every token.  Those roundings change from token to
// token and do not add up in one direction.  D itself is held as hi + lo
// (from an fp64 exp), since a fixed error in D would again act on every token
// alike.  The anchor moves:
//   - up to k, exactly, when a new key exceeds it (the history is rescaled
//     by e^{p-k} <= 1);
//   - down by kStepReanchor when the decayed sums fall below 2^-40, so that
//     new keys never underflow against a stale anchor.  This happens about
//     once every kStepReanchor / w tokens.
// The state is any (a, b, p) with the same e^p a and e^p b, so p need not be
// the running maximum.  GATED as in frame_token: gd = 1 + e^{-r}.
constexpr float kStepReanchor = 28.0f;                  // natural-log units
constexpr float kStepExpReanchor = 1.44625706e12f;      // e^28, rounded to fp32
constexpr float kStepLowSum = 9.094947e-13f;            // 2^-40

template <bool GATED = false>
__device__ __forceinline__ float decode_token(float& a, float& b, float& p, float k, float v,
                                              float w, float u, float gd = 1.0f) {
    const double dd = exp(-double(w));
    const float dhi = float(dd);
    const float dlo = float(dd - double(dhi));
    const float x = k - p;                   // new key against the anchor
    const float e = exp_neg_abs(x);
    const bool keep = x <= 0.0f;             // the anchor stays
    const float alpha = keep ? 1.0f : e;     // history moved to an anchor at k
    const float beta = keep ? e : 1.0f;      // weight of the new token
    float ta = alpha * a;
    float tb = alpha * b;
    ta = __builtin_fmaf(ta, dhi, ta * dlo);  // decayed by one token
    tb = __builtin_fmaf(tb, dhi, tb * dlo);
    const float wmu = w - u;
    float y;
    if (__builtin_fabsf(wmu) <= kFusedMaxAbsUW) {
        // read-out weights are the fold-in weights times (D, e^{u-w})
        const float delta = beta * __builtin_amdgcn_exp2f(-wmu * kLog2e);
        const float den = tb + delta;
        y = __builtin_fmaf(delta, v, ta) * fast_rcp(GATED ? den * gd : den);
    } else {
        // read-out as written: history at exponent p against u + k
        const float dr = -x - u;
        const float er = exp_neg_abs(dr);
        const bool kr = dr >= 0.0f;
        const float ar = kr ? 1.0f : er;
        const float br = kr ? er : 1.0f;
        const float den = __builtin_fmaf(ar, b, br);
        y = __builtin_fmaf(br, v, ar * a) * fast_rcp(GATED ? den * gd : den);
    }
    a = __builtin_fmaf(beta, v, ta);
    b = tb + beta;
    p = keep ? p : k;
    // downward re-anchor: p - 28 with its rounding error (TwoSum) folded
    // into the factor e^{28 + err} that a and b take
    const bool low = b < kStepLowSum;
    const float ps = p - kStepReanchor;
    const float z = ps - p;
    const float err = (p - (ps - z)) + (-kStepReanchor - z);
    const float f = __builtin_fmaf(kStepExpReanchor, err, kStepExpReanchor);
    a = low ? a * f : a;
    b = low ? b * f : b;
    p = low ? ps : p;
    return y;
}

__device__ __forceinline__ float clamp_empty(float p) { return p <= kEmptyIn ? kEmptyP : p; }
__device__ __forceinline__ float export_p(float p) { return p <= kEmptyIn ? -__builtin_inff() : p; }

// ---------------------------------------------------------------------------
// Storage of k, v, y: VEC consecutive channels per lane in one "raw" word.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    // v_cvt_pk_bf16_f32: round to nearest even
    f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
// Widening is recomputed at every use (the asm is opaque to common
// subexpression elimination): keeping the widened values of a whole chunk live
// between passes would double the registers the chunk occupies.
__device__ __forceinline__ float bf16_lo(uint32_t r) {
    uint32_t x;
    asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(x) : "v"(r));
    return __uint_as_float(x);
}
__device__ __forceinline__ float bf16_hi(uint32_t r) {
    uint32_t x;
    asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(x) : "v"(r));
    return __uint_as_float(x);
}

template <int DT, int VEC>
struct Io;

template <>
struct Io<kF32, 1> {
    using Raw = float;
    static __device__ __forceinline__ void unpack(Raw r, float (&x)[1]) { x[0] = r; }
    static __device__ __forceinline__ Raw pack(const float (&x)[1]) { return x[0]; }
    static __device__ __forceinline__ Raw zero() { return 0.0f; }
};

template <>
struct Io<kF32, 2> {
    using Raw = float2;
    static __device__ __forceinline__ void unpack(Raw r, float (&x)[2]) { x[0] = r.x; x[1] = r.y; }
    static __device__ __forceinline__ Raw pack(const float (&x)[2]) { return make_float2(x[0], x[1]); }
    static __device__ __forceinline__ Raw zero() { return make_float2(0.0f, 0.0f); }
};

template <>
struct Io<kF32, 4> {
    using Raw = float4;
    static __device__ __forceinline__ void unpack(Raw r, float (&x)[4]) {
        x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
    }
    static __device__ __forceinline__ Raw pack(const float (&x)[4]) {
        return make_float4(x[0], x[1], x[2], x[3]);
    }
    static __device__ __forceinline__ Raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};

template <>
struct Io<kBF16, 1> {
    using Raw = uint16_t;
    static __device__ __forceinline__ void unpack(Raw r, float (&x)[1]) {
        x[0] = __uint_as_float(uint32_t(r) << 16);
    }
    static __device__ __forceinline__ Raw pack(const float (&x)[1]) {
        return uint16_t(pack_bf16x2(x[0], 0.0f) & 0xffffu);
    }
    static __device__ __forceinline__ Raw zero() { return 0; }
};

template <>
struct Io<kBF16, 2> {
    using Raw = uint32_t;
    static __device__ __forceinline__ void unpack(Raw r, float (&x)[2]) {
        x[0] = bf16_lo(r);
        x[1] = bf16_hi(r);
    }
    static __device__ __forceinline__ Raw pack(const float (&x)[2]) { return pack_bf16x2(x[0], x[1]); }
    static __device__ __forceinline__ Raw zero() { return 0u; }
};

template <>
struct Io<kBF16, 4> {
    using Raw = uint2;
    static __device__ __forceinline__ void unpack(Raw r, float (&x)[4]) {
        x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x); x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
    }
    static __device__ __forceinline__ Raw pack(const float (&x)[4]) {
        return make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
    }
    static __device__ __forceinline__ Raw zero() { return make_uint2(0u, 0u); }
};

template <>
struct Io<kBF16, 8> {
    using Raw = uint4;
    static __device__ __forceinline__ void unpack(Raw r, float (&x)[8]) {
        x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x); x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
        x[4] = bf16_lo(r.z); x[5] = bf16_hi(r.z); x[6] = bf16_lo(r.w); x[7] = bf16_hi(r.w);
    }
    static __device__ __forceinline__ Raw pack(const float (&x)[8]) {
        return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                          pack_bf16x2(x[6], x[7]));
    }
    static __device__ __forceinline__ Raw zero() { return make_uint4(0u, 0u, 0u, 0u); }
};

// ---------------------------------------------------------------------------
// Buffer addressing: a wave-uniform base in a buffer resource (SGPRs), a
// per-lane byte offset (VGPR, fixed for the kernel) and a per-token byte
// offset (SGPR).  Address arithmetic then costs no vector instructions.
// ---------------------------------------------------------------------------

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer (stride 0) covering 4 GiB from `base`; dword 3 selects 32-bit
// data format, as required by untyped buffer instructions on gfx9.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// Cache policies of the k, v loads: non-temporal (each word is read once),
// which streams the strip-per-workgroup pattern of the serial and chained
// token loops at a markedly higher rate on MI355X, and the default one,
// which the chunked path's tiles measure faster with.
constexpr int kStreamLoad = 2;
constexpr int kDefaultLoad = 0;

// Cache policies of the stores: the default one, and device scope (sc1),
// which writes through the XCD's L2 instead of leaving dirty lines there to
// be evicted among the reads.  The streams written once measure faster with
// it: the forward's y (the bf16 workload's chained kernel 153.7 -> 147.9 us
// over 500 launches) and the matrix-state forward's y tiles.  The
// backward's gk, gv, the token shift's three outputs and the decode steps'
// y and state go fastest with non-temporal stores instead.
constexpr int kStreamStore = 16;
constexpr int kDefaultStore = 0;
// Non-temporal stores: the backward's gk, gv (362 -> 339 us for the
// saved-state backward on the bf16 workload; sc1 measured 364 us there).
constexpr int kNonTemporalStore = 2;

// A non-temporal load through a plain pointer (2, 4, 8 or 16 bytes), for
// the elementwise kernels' once-read inputs.
template <typename T>
__device__ __forceinline__ T load_stream(const T* p) {
    if constexpr (sizeof(T) == 2)
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p)));
    else if constexpr (sizeof(T) == 4)
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)));
    else if constexpr (sizeof(T) == 8)
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p)));
    else
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

// A non-temporal store through a plain pointer (2, 4, 8 or 16 bytes).
template <typename T>
__device__ __forceinline__ void store_stream(T* p, T x) {
    if constexpr (sizeof(T) == 2)
        __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, x), reinterpret_cast<uint16_t*>(p));
    else if constexpr (sizeof(T) == 4)
        __builtin_nontemporal_store(__builtin_bit_cast(uint32_t, x), reinterpret_cast<uint32_t*>(p));
    else if constexpr (sizeof(T) == 8)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x2_t, x), reinterpret_cast<u32x2_t*>(p));
    else
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, x), reinterpret_cast<u32x4_t*>(p));
}

template <typename Raw>
struct Buf;

template <>
struct Buf<float> {
    template <int AUX = kStreamLoad>
    static __device__ __forceinline__ float load(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
    }
    template <int AUX = kDefaultStore>
    static __device__ __forceinline__ void store(float x, rsrc_t r, uint32_t voff, uint32_t soff) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, voff, soff, AUX);
    }
};
template <>
struct Buf<uint32_t> {
    template <int AUX = kStreamLoad>
    static __device__ __forceinline__ uint32_t load(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX);
    }
    template <int AUX = kDefaultStore>
    static __device__ __forceinline__ void store(uint32_t x, rsrc_t r, uint32_t voff, uint32_t soff) {
        __builtin_amdgcn_raw_buffer_store_b32(x, r, voff, soff, AUX);
    }
};
template <>
struct Buf<uint16_t> {
    template <int AUX = kStreamLoad>
    static __device__ __forceinline__ uint16_t load(rsrc_t r, uint32_t voff, uint32_t soff) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, AUX);
    }
    template <int AUX = kDefaultStore>
    static __device__ __forceinline__ void store(uint16_t x, rsrc_t r, uint32_t voff, uint32_t soff) {
        __builtin_amdgcn_raw_buffer_store_b16(x, r, voff, soff, AUX);
    }
};
template <>
struct Buf<float2> {
    template <int AUX = kStreamLoad>
    static __device__ __forceinline__ float2 load(rsrc_t r, uint32_t voff, uint32_t soff) {
        const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
        return make_float2(__uint_as_float(x.x), __uint_as_float(x.y));
    }
    template <int AUX = kDefaultStore>
    static __device__ __forceinline__ void store(float2 x, rsrc_t r, uint32_t voff, uint32_t soff) {
        const u32x2_t v = {__float_as_uint(x.x), __float_as_uint(x.y)};
        __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, AUX);
    }
};
template <>
struct Buf<uint2> {
    template <int AUX = kStreamLoad>
    static __device__ __forceinline__ uint2 load(rsrc_t r, uint32_t voff, uint32_t soff) {
        const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
        return make_uint2(x.x, x.y);
    }
    template <int AUX = kDefaultStore>
    static __device__ __forceinline__ void store(uint2 x, rsrc_t r, uint32_t voff, uint32_t soff) {
        const u32x2_t v = {x.x, x.y};
        __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, AUX);
    }
};
template <>
struct Buf<float4> {
    template <int AUX = kStreamLoad>
    static __device__ __forceinline__ float4 load(rsrc_t r, uint32_t voff, uint32_t soff) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
        return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                           __uint_as_float(x.w));
    }
    template <int AUX = kDefaultStore>
    static __device__ __forceinline__ void store(float4 x, rsrc_t r, uint32_t voff, uint32_t soff) {
        const u32x4_t v = {__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z),
                           __float_as_uint(x.w)};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, AUX);
    }
};

// ---------------------------------------------------------------------------
// Cross-workgroup publication of partial states.
//
// Data words are written with agent-scope relaxed atomic stores and read with
// agent-scope relaxed atomic loads: those are coherent across the chip's
// XCDs without flushing or invalidating the L2.  A publisher orders its data
// before its flag by waiting for all of its outstanding memory operations
// (s_waitcnt vmcnt(0)) before the flag store; a reader issues its data loads
// only after its flag load has returned the expected value.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void st_agent(float* p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint64_t* p, uint64_t x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_flag(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave has issued has completed.
__device__ __forceinline__ void wait_all_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Keep the compiler from moving memory operations across this point.
__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

}  // namespace wkv
