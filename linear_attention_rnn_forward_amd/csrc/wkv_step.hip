// wkv_step: one decode token for every (layer, sequence, channel) of [L,S,C]
// ([aiwiki] = aiwiki.thehackersbrain.dev rwkv, the wkv_step listing: state
// (a, b, p) in, output and new state out; [multigrid] = multigrid.ai rwkv,
// "Prefill, decode, and where each form is used").
//
// Purely elementwise: every element reads k, v, a, b, p and writes y, a', b',
// p'.  VEC adjacent channels per lane with vector loads.  The per-element
// arithmetic is decode_token() from wkv_device.h: natural-log exponents, the
// exponent held as an anchor that moves only to an exact new maximum (or
// rarely down), and the decay applied to a, b as e^{-w} in hi + lo parts, so
// that no rounding repeats the same way token after token.
#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

template <int VEC>
struct F32v;
template <>
struct F32v<1> {
    using T = float;
    static __device__ __forceinline__ void get(T r, float (&x)[1]) { x[0] = r; }
    static __device__ __forceinline__ T put(const float (&x)[1]) { return x[0]; }
};
template <>
struct F32v<4> {
    using T = float4;
    static __device__ __forceinline__ void get(T r, float (&x)[4]) {
        x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
    }
    static __device__ __forceinline__ T put(const float (&x)[4]) { return make_float4(x[0], x[1], x[2], x[3]); }
};

// GATED: y = sigmoid(r) * wkv (the receptance gate, [tm-math] "Receptance:
// the gate on the way out").
template <int DT, int VEC, bool GATED>
__global__ __launch_bounds__(256) void step_kernel(StepProblem pr, int64_t nvec) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    using FV = F32v<VEC>;
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= nvec) return;
    const int64_t e0 = i * VEC;                 // first element
    const int64_t l = e0 / (pr.S * pr.C);
    const int64_t c = e0 % pr.C;
    const float* wp = pr.w + l * pr.C + c;
    const float* up = pr.u + l * pr.C + c;

    float kf[VEC], vf[VEC], a[VEC], b[VEC], p[VEC], y[VEC], rf[VEC];
    IO::unpack(load_stream(reinterpret_cast<const Raw*>(pr.k) + i), kf);
    IO::unpack(load_stream(reinterpret_cast<const Raw*>(pr.v) + i), vf);
    FV::get(load_stream(reinterpret_cast<const typename FV::T*>(pr.a_in) + i), a);
    FV::get(load_stream(reinterpret_cast<const typename FV::T*>(pr.b_in) + i), b);
    FV::get(load_stream(reinterpret_cast<const typename FV::T*>(pr.p_in) + i), p);
    if constexpr (GATED) IO::unpack(load_stream(reinterpret_cast<const Raw*>(pr.r) + i), rf);
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        p[q] = clamp_empty(p[q]);
        y[q] = decode_token<GATED>(a[q], b[q], p[q], kf[q], vf[q], wp[q], up[q],
                                   GATED ? gate_den(rf[q]) : 1.0f);
        p[q] = export_p(p[q]);
    }
    // the outputs through plain non-temporal stores (209.4 us on the decode
    // workload, against 220.5 with default stores and 210.0 with device-scope
    // buffer stores)
    store_stream(reinterpret_cast<Raw*>(pr.y) + i, IO::pack(y));
    store_stream(reinterpret_cast<typename FV::T*>(pr.a_out) + i, FV::put(a));
    store_stream(reinterpret_cast<typename FV::T*>(pr.b_out) + i, FV::put(b));
    store_stream(reinterpret_cast<typename FV::T*>(pr.p_out) + i, FV::put(p));
}

}  // namespace

namespace {
template <bool GATED>
void launch_step_t(const StepProblem& pr, int64_t nvec, hipStream_t stream) {
    const int64_t blocks = (nvec + 255) / 256;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    if (pr.dtype == kBF16 && pr.vec == 4)
        hipLaunchKernelGGL((step_kernel<kBF16, 4, GATED>), grid, block, 0, stream, pr, nvec);
    else if (pr.dtype == kBF16)
        hipLaunchKernelGGL((step_kernel<kBF16, 1, GATED>), grid, block, 0, stream, pr, nvec);
    else if (pr.vec == 4)
        hipLaunchKernelGGL((step_kernel<kF32, 4, GATED>), grid, block, 0, stream, pr, nvec);
    else
        hipLaunchKernelGGL((step_kernel<kF32, 1, GATED>), grid, block, 0, stream, pr, nvec);
}
}  // namespace

hipError_t launch_step(const StepProblem& pr, hipStream_t stream) {
    const int64_t nvec = pr.L * pr.S * pr.C / pr.vec;
    if (pr.r != nullptr)
        launch_step_t<true>(pr, nvec, stream);
    else
        launch_step_t<false>(pr, nvec, stream);
    return hipGetLastError();
}

}  // namespace wkv
