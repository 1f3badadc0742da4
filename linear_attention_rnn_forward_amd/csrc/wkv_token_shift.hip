// Token shift: the two-tap causal lerp in front of the R, K, V projections
// ([tm-math] = aicassindra.com tm_rwkv_math, "Token shift: a two-tap causal
// convolution"; [multigrid] = multigrid.ai rwkv, "Token shift and channel
// mixing"), for the three blends mu_r, mu_k, mu_v in one pass over x:
//
//   xbar_t = mu * x_t + (1 - mu) * x_{t-1},  evaluated as x_{t-1} + mu * (x_t - x_{t-1})
//
// Each lane owns VEC adjacent channels of one batch row and a run of
// kShiftTokens consecutive tokens; it reads the token before its run once and
// then carries x_{t-1} in registers, so x is read once (plus one row per run)
// and the three outputs are written once.
#include "wkv_device.h"
#include "wkv_internal.h"

namespace wkv {
namespace {

template <int DT, int VEC>
__global__ __launch_bounds__(256) void token_shift_kernel(ShiftProblem pr, int64_t lanes_per_row,
                                                          int64_t runs) {
    using IO = Io<DT, VEC>;
    using Raw = typename IO::Raw;
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = pr.B * runs * lanes_per_row;
    if (i >= total) return;
    const int64_t cl = i % lanes_per_row;          // lane within the row
    const int64_t r = (i / lanes_per_row) % runs;  // run along T
    const int64_t bb = i / (lanes_per_row * runs);
    const int64_t c = cl * VEC;
    const int64_t t0 = r * kShiftTokens;
    const int64_t t1 = (t0 + kShiftTokens < pr.T) ? t0 + kShiftTokens : pr.T;

    float mr[VEC], mk[VEC], mv[VEC];
#pragma unroll
    for (int q = 0; q < VEC; q++) {
        mr[q] = pr.mu_r[c + q];
        mk[q] = pr.mu_k[c + q];
        mv[q] = pr.mu_v[c + q];
    }
    const Raw* x = reinterpret_cast<const Raw*>(pr.x);
    Raw* xr = reinterpret_cast<Raw*>(pr.xr);
    Raw* xk = reinterpret_cast<Raw*>(pr.xk);
    Raw* xv = reinterpret_cast<Raw*>(pr.xv);
    float prev[VEC];
    if (t0 > 0) {
        IO::unpack(x[(bb * pr.T + t0 - 1) * lanes_per_row + cl], prev);
    } else if (pr.x_prev != nullptr) {
        IO::unpack(reinterpret_cast<const Raw*>(pr.x_prev)[bb * lanes_per_row + cl], prev);
    } else {
#pragma unroll
        for (int q = 0; q < VEC; q++) prev[q] = 0.0f;
    }
    for (int64_t t = t0; t < t1; t++) {
        const int64_t idx = (bb * pr.T + t) * lanes_per_row + cl;
        float cur[VEC], orr[VEC], ok[VEC], ov[VEC];
        // default cache policy: each run's first token re-reads the row before
        // it, read by the neighbouring run (non-temporal loads: 193.7 against
        // 159.9 us on the bf16 workload)
        IO::unpack(x[idx], cur);
#pragma unroll
        for (int q = 0; q < VEC; q++) {
            const float d = cur[q] - prev[q];
            orr[q] = __builtin_fmaf(mr[q], d, prev[q]);
            ok[q] = __builtin_fmaf(mk[q], d, prev[q]);
            ov[q] = __builtin_fmaf(mv[q], d, prev[q]);
            prev[q] = cur[q];
        }
        // written once and not read back here: non-temporal stores
        store_stream(xr + idx, IO::pack(orr));
        store_stream(xk + idx, IO::pack(ok));
        store_stream(xv + idx, IO::pack(ov));
    }
    if (t1 == pr.T && pr.x_last != nullptr)
        reinterpret_cast<Raw*>(pr.x_last)[bb * lanes_per_row + cl] = IO::pack(prev);
}

// T == 0: x_last = x_prev or 0.
template <int DT>
__global__ void shift_last_only_kernel(ShiftProblem pr) {
    using IO = Io<DT, 1>;
    using Raw = typename IO::Raw;
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= pr.B * pr.C) return;
    Raw v = IO::zero();
    if (pr.x_prev != nullptr) v = reinterpret_cast<const Raw*>(pr.x_prev)[i];
    reinterpret_cast<Raw*>(pr.x_last)[i] = v;
}

template <int DT, int VEC>
hipError_t launch_vec(const ShiftProblem& pr, hipStream_t stream) {
    const int64_t lanes_per_row = pr.C / VEC;
    const int64_t runs = (pr.T + kShiftTokens - 1) / kShiftTokens;
    const int64_t total = pr.B * runs * lanes_per_row;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL((token_shift_kernel<DT, VEC>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                       pr, lanes_per_row, runs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_token_shift(const ShiftProblem& pr, hipStream_t stream) {
    if (pr.T == 0) {
        if (pr.x_last == nullptr) return hipSuccess;
        const int64_t blocks = (pr.B * pr.C + 255) / 256;
        if (pr.dtype == kBF16)
            hipLaunchKernelGGL(shift_last_only_kernel<kBF16>, dim3(unsigned(blocks)), dim3(256), 0, stream, pr);
        else
            hipLaunchKernelGGL(shift_last_only_kernel<kF32>, dim3(unsigned(blocks)), dim3(256), 0, stream, pr);
        return hipGetLastError();
    }
    if (pr.dtype == kBF16) {
        if (pr.vec == 8) return launch_vec<kBF16, 8>(pr, stream);
        if (pr.vec == 4) return launch_vec<kBF16, 4>(pr, stream);
        if (pr.vec == 2) return launch_vec<kBF16, 2>(pr, stream);
        return launch_vec<kBF16, 1>(pr, stream);
    }
    if (pr.vec == 4) return launch_vec<kF32, 4>(pr, stream);
    return launch_vec<kF32, 1>(pr, stream);
}

}  // namespace wkv
