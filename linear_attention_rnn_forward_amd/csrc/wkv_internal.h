// Host-side interface between the C ABI layer (wkv_api.hip) and the kernel
// launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "wkv.h"

namespace wkv {

struct ForwardProblem {
    int64_t B, T, C;
    int dtype;
    int vec;                          // channels per lane (from pick_forward_vec)
    const float *w, *u;
    const void *k, *v;
    void *y;
    const float *a_in, *b_in, *p_in;  // all null or all set
    float *a_out, *b_out, *p_out;     // all null or all set
    const void* r = nullptr;          // receptance [B,T,C]: y = sigmoid(r) * wkv when set
    float* states = nullptr;          // [B][ceil(T/16)][4][C]: the chained path's carries, when set
};

// Geometry of the chunked path for one problem.
struct ChunkPlan {
    int vec;                 // channels per lane
    int64_t ngroups;         // column groups: B * ceil(C / (64 * vec))
    int64_t tiles_per_group; // ceil(T / tile_tokens)
    int waves;               // waves per tile (workgroup)
    int tile_tokens;         // tokens per workgroup tile
    size_t workspace_bytes;
};

// Which path wkv_forward takes for a problem (never returns WKV_PATH_AUTO).
int choose_forward_path(const ForwardProblem& pr, int device_cus);
// waves: 0 to choose from the problem and the current device, else the
// waves per tile to plan for.
ChunkPlan plan_chunked(int64_t B, int64_t T, int64_t C, int vec, int waves = 0);
// Channels per lane for wkv_forward: 2 for bf16 when C is even and k, v, y
// are 4-byte aligned, else 1.
int pick_forward_vec(int64_t C, int dtype, bool aligned);
size_t forward_workspace_bytes(int64_t B, int64_t T, int64_t C, int dtype, int path);

hipError_t launch_forward_serial(const ForwardProblem& pr, hipStream_t stream);
hipError_t launch_forward_chunked(const ForwardProblem& pr, void* workspace, hipStream_t stream);
hipError_t launch_forward_chained(const ForwardProblem& pr, hipStream_t stream);
// T == 0: state_out = state_in (or the empty state).
hipError_t launch_state_passthrough(const ForwardProblem& pr, hipStream_t stream);
// Bounded waits that gave up on the current device since the library was
// loaded: the chunked forward's look-back, the matrix forward's ring.
hipError_t read_chunk_wait_failures(uint64_t* count);
hipError_t read_ring_wait_failures(uint64_t* count);

struct StepProblem {
    int64_t L, S, C;
    int dtype;
    int vec;  // 4 when C % 4 == 0 and every array is 16-byte aligned, else 1
    const float *w, *u;
    const void *k, *v;
    void *y;
    const float *a_in, *b_in, *p_in;
    float *a_out, *b_out, *p_out;
    const void* r = nullptr;  // receptance [L,S,C]: y = sigmoid(r) * wkv when set
};
hipError_t launch_step(const StepProblem& pr, hipStream_t stream);

// Gradients of sum(gy * wkv) for wkv_forward from the empty history.
struct BackwardProblem {
    int64_t B, T, C;
    int dtype;
    const float *w, *u;
    const void *k, *v, *gy;        // [B,T,C] dtype
    void *gk, *gv;                 // [B,T,C] dtype
    float *gw, *gu;                // [C]
    int vec = 1;                   // channels per lane (backward_vec)
    // workspace sections (set by launch_backward)
    const float* saved = nullptr;  // [B][ceil(T/16)][4][C] checkpoints saved by the forward, or null
    float* ckpt = nullptr;         // [B][ceil(T/16)][4][C] forward state before each sub-chunk
    float* part_w = nullptr;       // [B,C] per-column gw
    float* part_u = nullptr;       // [B,C] per-column gu
};
int backward_vec(int64_t C, int dtype, bool aligned);
size_t backward_workspace_bytes(int64_t B, int64_t T, int64_t C, bool saved);
hipError_t launch_backward(BackwardProblem pr, void* workspace, hipStream_t stream);

// Tokens per lane in the token shift: each lane reads the row before its run
// once more, so short runs cost 1/kShiftTokens of x again but give the
// stream many more independent lanes (8 measured fastest on the bf16 [16,
// 4096, 2048] shift among 4..64).
constexpr int kShiftTokens = 8;

struct ShiftProblem {
    int64_t B, T, C;
    int dtype;
    int vec;  // 8 (bf16 only), 4, 2 or 1 channels per lane, dividing C, arrays aligned for it
    const void *x, *x_prev;
    const float *mu_r, *mu_k, *mu_v;
    void *xr, *xk, *xv, *x_last;
};
hipError_t launch_token_shift(const ShiftProblem& pr, hipStream_t stream);

// Matrix-valued state WKV (RWKV-5/6): head dimension 64, C = 64 H.
struct MatProblem {
    int64_t B, T, H;
    int dtype;
    const void *r, *k, *v;   // [B,T,C] dtype
    const void* z;           // [B,T,C] dtype when z_per_token, else [C] fp32
    int z_per_token;
    const float* s_in;       // [B,H,64,64] fp32 or null (zero state)
    float* s_out;            // [B,H,64,64] fp32 or null
    void* y;                 // [B,T,C] dtype
    int path;                // 0: chunked matrix-core form (bf16), 1: token by token
};
hipError_t launch_mat_forward(const MatProblem& pr, hipStream_t stream);

struct MatStepProblem {
    int64_t L, S, H;
    int dtype;
    const void *r, *k, *v;   // [L,S,C] dtype
    const void* z;           // [L,S,C] dtype when z_per_token, else [L,C] fp32
    int z_per_token;
    const float* s_in;       // [L,S,H,64,64] fp32
    float* s_out;            // same shape; may equal s_in
    void* y;                 // [L,S,C] dtype
};
hipError_t launch_mat_step(const MatStepProblem& pr, hipStream_t stream);

int device_cu_count();  // CUs of the current device (cached per device)

}  // namespace wkv
