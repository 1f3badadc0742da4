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
// gy_t y_t (a scan backwards in time: P_{i-1} = gy_i / D_i + e^{-w} P_i), and
// A'_t, B'_t the history sums weighted by their age t-1-i (a scan forwards:
// A'_{t+1} = e^{-w} (A'_t + A_t)).  gw and gu are summed over B and T.
//
// Two passes per column (b, c), one lane per column:
//   1. forward in t: the stabilised state (a, b, a', b') with exponent p,
//      kept as an anchor and a token count (p = A - m w, one rounding per
//      token, none accumulated); writes z_t = log D_t and y_t (fp32) to the
//      workspace and accumulates the column's gw, gu terms;
//   2. backward in t: (P, Q) scaled by e^{pi}, pi kept the same way as an
//      anchor and a count; writes gk, gv.
// Every exponential has a non-positive argument: p <= z_t, k_i + pi <= 0
// (D_t contains token i's own weight), u + k_t <= z_t.
// A final kernel sums the per-column gw, gu over the batch in a fixed order.
#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

constexpr int kBwdTokens = 16;  // tokens loaded ahead per lane

__device__ __forceinline__ float expf_(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float logf_(float x) { return __builtin_amdgcn_logf(x) * 0.69314718055994531f; }

template <int DT>
__global__ __launch_bounds__(256) void backward_forward_pass(BackwardProblem pr) {
    using IO = Io<DT, 1>;
    using Raw = typename IO::Raw;
    const int64_t col = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (col >= pr.B * pr.C) return;
    const int64_t bb = col / pr.C;
    const int64_t c = col - bb * pr.C;
    const int64_t T = pr.T, C = pr.C;
    const float w = pr.w[c], u = pr.u[c];
    const Raw* kp = static_cast<const Raw*>(pr.k) + bb * T * C + c;
    const Raw* vp = static_cast<const Raw*>(pr.v) + bb * T * C + c;
    const Raw* gp = static_cast<const Raw*>(pr.gy) + bb * T * C + c;
    float* zp = pr.z + bb * T * C + c;
    float* yp = pr.ys + bb * T * C + c;

    float A = kEmptyP, m = 0.0f;              // history exponent p = A - m w
    float a = 0.0f, b = 0.0f, ap = 0.0f, bp = 0.0f;
    float gw = 0.0f, gu = 0.0f;
    for (int64_t t0 = 0; t0 < T; t0 += kBwdTokens) {
        const int n = T - t0 < kBwdTokens ? int(T - t0) : kBwdTokens;
        float kf[kBwdTokens], vf[kBwdTokens], gf[kBwdTokens];
#pragma unroll
        for (int i = 0; i < kBwdTokens; i++) {
            if (i < n) {
                float x[1];
                IO::unpack(load_stream(kp + (t0 + i) * C), x); kf[i] = x[0];
                IO::unpack(load_stream(vp + (t0 + i) * C), x); vf[i] = x[0];
                IO::unpack(load_stream(gp + (t0 + i) * C), x); gf[i] = x[0];
            }
        }
#pragma unroll
        for (int i = 0; i < kBwdTokens; i++) {
            if (i < n) {
                const float k = kf[i], v = vf[i], g = gf[i];
                // exponent differences are formed anchor-relative: A - k is
                // exact when the two are close (Sterbenz) and the m w term is
                // added by one fma at the difference's own magnitude, so the
                // per-token rescalings carry no rounding of |k| ~ 100
                const float ak = A - k;
                const float d = __builtin_fmaf(-m, w, ak - u);       // p - (u + k)
                const float al = expf_(min_num(d, 0.0f));             // e^{p - q}
                const float be = expf_(min_num(-d, 0.0f));            // e^{u + k - q}
                const float del = __builtin_fmaf(al, b, be);
                const float y = __builtin_fmaf(al, a, be * v) * fast_rcp(del);
                const float ld = logf_(del);
                const float q = d >= 0.0f ? __builtin_fmaf(-m, w, A) : u + k;
                zp[(t0 + i) * C] = q + ld;
                yp[(t0 + i) * C] = y;
                // this token's terms of gu and gw (1/D_t = e^{-z_t})
                gu = __builtin_fmaf(g * expf_(min_num(-d, 0.0f) - ld), v - y, gu);
                gw = __builtin_fmaf(-g * expf_(min_num(d, 0.0f) - ld), __builtin_fmaf(-y, bp, ap), gw);
                // fold token t in: the history decays by e^{-w}, the age-weighted
                // sums gain the history, the new key enters with weight e^{k};
                // e = (p - w) - k
                const float e = __builtin_fmaf(-(m + 1.0f), w, ak);
                if (e < 0.0f) {
                    const float s = expf_(e);
                    ap = s * (ap + a);
                    bp = s * (bp + b);
                    a = __builtin_fmaf(s, a, v);
                    b = __builtin_fmaf(s, b, 1.0f);
                    A = k;
                    m = 0.0f;
                } else {
                    const float s = expf_(-e);
                    ap += a;
                    bp += b;
                    a = __builtin_fmaf(s, v, a);
                    b += s;
                    m += 1.0f;
                }
            }
        }
    }
    pr.part_w[col] = gw;
    pr.part_u[col] = gu;
}

template <int DT>
__global__ __launch_bounds__(256) void backward_reverse_pass(BackwardProblem pr) {
    using IO = Io<DT, 1>;
    using Raw = typename IO::Raw;
    const int64_t col = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (col >= pr.B * pr.C) return;
    const int64_t bb = col / pr.C;
    const int64_t c = col - bb * pr.C;
    const int64_t T = pr.T, C = pr.C;
    const float w = pr.w[c], u = pr.u[c];
    const Raw* kp = static_cast<const Raw*>(pr.k) + bb * T * C + c;
    const Raw* vp = static_cast<const Raw*>(pr.v) + bb * T * C + c;
    const Raw* gp = static_cast<const Raw*>(pr.gy) + bb * T * C + c;
    const float* zp = pr.z + bb * T * C + c;
    const float* yp = pr.ys + bb * T * C + c;
    Raw* gkp = static_cast<Raw*>(pr.gk) + bb * T * C + c;
    Raw* gvp = static_cast<Raw*>(pr.gv) + bb * T * C + c;

    float Pi = kEmptyP, n = 0.0f;             // scale exponent pi = Pi - n w (anchor Pi = -z)
    float P = 0.0f, Q = 0.0f;
    for (int64_t t1 = T; t1 > 0; t1 -= kBwdTokens) {
        const int cnt = t1 < kBwdTokens ? int(t1) : kBwdTokens;
        const int64_t t0 = t1 - cnt;
        float kf[kBwdTokens], vf[kBwdTokens], gf[kBwdTokens], zf[kBwdTokens], yf[kBwdTokens];
#pragma unroll
        for (int i = 0; i < kBwdTokens; i++) {
            if (i < cnt) {
                float x[1];
                IO::unpack(load_stream(kp + (t0 + i) * C), x); kf[i] = x[0];
                IO::unpack(load_stream(vp + (t0 + i) * C), x); vf[i] = x[0];
                IO::unpack(load_stream(gp + (t0 + i) * C), x); gf[i] = x[0];
                zf[i] = load_stream(zp + (t0 + i) * C);
                yf[i] = load_stream(yp + (t0 + i) * C);
            }
        }
#pragma unroll
        for (int i = kBwdTokens - 1; i >= 0; i--) {
            if (i < cnt) {
                const float k = kf[i], v = vf[i], g = gf[i], z = zf[i], y = yf[i];
                // gy_t e^{u+k_t} / D_t; u + k rounds as where z was formed, so
                // the exponent is exactly -log(delta) when the bonus dominates
                const float ed = g * expf_((u + k) - z);
                const float eh = expf_(__builtin_fmaf(-n, w, k + Pi)); // e^{k_t} times the scale of P, Q
                float gv[1], gk[1];
                gv[0] = __builtin_fmaf(eh, P, ed);
                gk[0] = __builtin_fmaf(eh, __builtin_fmaf(v, P, -Q), ed * (v - y));
                gvp[(t0 + i) * C] = IO::pack(gv);
                gkp[(t0 + i) * C] = IO::pack(gk);
                // fold token t into P, Q for the earlier tokens; the new term's
                // exponent is -z_t, e = (pi - w) - (-z_t), anchor-relative
                const float e = __builtin_fmaf(-(n + 1.0f), w, Pi + z);
                if (e < 0.0f) {
                    const float s = expf_(e);
                    P = __builtin_fmaf(s, P, g);
                    Q = __builtin_fmaf(s, Q, g * y);
                    Pi = -z;
                    n = 0.0f;
                } else {
                    const float s = expf_(-e);
                    P = __builtin_fmaf(s, g, P);
                    Q = __builtin_fmaf(s * g, y, Q);
                    n += 1.0f;
                }
            }
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

}  // namespace

size_t backward_workspace_bytes(int64_t B, int64_t T, int64_t C) {
    const size_t n = size_t(B) * size_t(T) * size_t(C);
    const size_t cols = size_t(B) * size_t(C);
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    return up(n * 4) * 2 + up(cols * 4) * 2;
}

hipError_t launch_backward(BackwardProblem pr, void* workspace, hipStream_t stream) {
    const int64_t cols = pr.B * pr.C;
    if (pr.T == 0) {
        hipLaunchKernelGGL(zero_pair, dim3(unsigned((pr.C + 255) / 256)), dim3(256), 0, stream, pr.gw,
                           pr.gu, pr.C);
        return hipGetLastError();
    }
    const size_t n = size_t(pr.B) * size_t(pr.T) * size_t(pr.C);
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    char* ws = static_cast<char*>(workspace);
    pr.z = reinterpret_cast<float*>(ws);
    pr.ys = reinterpret_cast<float*>(ws + up(n * 4));
    pr.part_w = reinterpret_cast<float*>(ws + 2 * up(n * 4));
    pr.part_u = reinterpret_cast<float*>(ws + 2 * up(n * 4) + up(size_t(cols) * 4));
    const dim3 grid(unsigned((cols + 255) / 256)), block(256);
    if (pr.dtype == kBF16) {
        hipLaunchKernelGGL(backward_forward_pass<kBF16>, grid, block, 0, stream, pr);
        hipLaunchKernelGGL(backward_reverse_pass<kBF16>, grid, block, 0, stream, pr);
    } else {
        hipLaunchKernelGGL(backward_forward_pass<kF32>, grid, block, 0, stream, pr);
        hipLaunchKernelGGL(backward_reverse_pass<kF32>, grid, block, 0, stream, pr);
    }
    hipLaunchKernelGGL(backward_reduce, dim3(unsigned((pr.C + 255) / 256)), dim3(256), 0, stream, pr);
    return hipGetLastError();
}

}  // namespace wkv
