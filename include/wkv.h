/*
 * wkv.h -- C ABI of libwkv: the RWKV-4 WKV operator on AMD MI355X (gfx950).
 *
 * Sources for what the operator computes (cited by page and section):
 *   [aiwiki]    aiwiki.thehackersbrain.dev/entries/rwkv -- "RWKV", the wkv_step
 *               listing and the note under it
 *   [tm-math]   aicassindra.com/blogs/transformer_math/tm_rwkv_math.html --
 *               "The WKV operator: attention with a fixed decay", "Why it
 *               collapses into a recurrence", "Numerical stability: carry the
 *               exponent", "Token shift: a two-tap causal convolution"
 *   [vanos]     vanos001.github.io/placement_prep/llm/architectures/rwkv.html --
 *               "The WKV Operator: Attention and RNN at Once"
 *   [multigrid] multigrid.ai/learn/rwkv -- "Prefill, decode, and where each
 *               form is used", "The state, in bytes"
 *
 * Definition ([tm-math] "The WKV operator"), per batch row b and channel c,
 * tokens counted from 0:
 *
 *   y_t = ( sum_{i<t} e^{-(t-1-i) w + k_i} v_i + e^{u + k_t} v_t )
 *       / ( sum_{i<t} e^{-(t-1-i) w + k_i}     + e^{u + k_t}     )
 *
 * with w > 0 the per-channel decay rate and u the current-token bonus.  It is
 * evaluated by the max-stabilised recurrence on a state (a, b, p) whose true
 * accumulators are e^p a and e^p b ([tm-math] "Numerical stability"; [aiwiki]
 * wkv_step).  The empty history is a = b = 0, p = -inf.
 *
 * Conventions shared by every call:
 *   - All array pointers are DEVICE pointers, owned by the caller.  The
 *     library never allocates, frees or keeps a pointer after returning.
 *   - Arrays are dense and row-major ("C-contiguous"); shapes are given in
 *     each call's comment.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls validate their
 *     arguments on the host, enqueue work on `stream` and return without
 *     synchronising.  A nonzero return means nothing was enqueued, except
 *     WKV_ERR_HIP, which reports a launch failure.
 *   - Errors are negative wkv_status codes; wkv_last_error() gives a message
 *     for the last failing call on the calling thread.
 *   - Floating-point results are fp32 arithmetic; bf16 outputs are rounded
 *     to nearest-even.  p arguments are in natural-log units.  On input any
 *     p <= -1e30 (including -inf) means "empty"; an empty state is returned
 *     as p = -inf.
 *   - Non-finite inputs are outside the contract.
 *   - w <= 0 is outside the contract ([tm-math] states w = exp(omega) > 0);
 *     it is not checked.
 */
#ifndef WKV_H
#define WKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of k, v, y (and of x, xr, xk, xv in wkv_token_shift).
 * w, u and the state are always fp32. */
typedef enum {
    WKV_F32 = 0,
    WKV_BF16 = 1
} wkv_dtype;

typedef enum {
    WKV_OK = 0,
    WKV_ERR_NULL = -1,        /* a required pointer is NULL                       */
    WKV_ERR_SHAPE = -2,       /* a size is negative / zero where not allowed,     */
                              /* or a product overflows int64                     */
    WKV_ERR_DTYPE = -3,       /* unknown wkv_dtype                                */
    WKV_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than the size query    */
    WKV_ERR_ALIAS = -5,       /* an output overlaps an input it may not overlap   */
    WKV_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed       */
    WKV_ERR_UNSUPPORTED = -7, /* an option this build does not provide            */
    WKV_ERR_ARG = -8          /* an argument out of its documented range          */
} wkv_status;

/* Execution path for wkv_forward_path(). */
typedef enum {
    WKV_PATH_AUTO = 0,        /* chosen from B*C, T and the device's CU count     */
    WKV_PATH_SERIAL = 1,      /* one lane per (b, channel group), scan along T    */
    WKV_PATH_CHUNKED = 2,     /* time-parallel tiles on separate workgroups; partial   */
                              /* states passed through the workspace                   */
    WKV_PATH_CHAINED = 3      /* one workgroup per channel group; its waves take       */
                              /* consecutive sub-chunks and pass the carry through LDS */
} wkv_path;

/* Bytes of device workspace wkv_forward needs for these sizes on the current
 * device (0 when the chosen path needs none).  Returns 0 for invalid sizes.
 * Only the chunked path (WKV_PATH_CHUNKED, chosen when B*C is too small to
 * occupy the device otherwise) uses one: per-tile partial states, flags and a
 * tile counter.  Its contents on entry do not matter: each call clears what it
 * uses with a kernel of its own (no memset node), so calls may be recorded in
 * a HIP graph and replayed.  Calls that share a workspace must be ordered on
 * one stream. */
size_t wkv_forward_workspace_size(int64_t B, int64_t T, int64_t C, int dtype);

/* Same, for an explicitly chosen path. */
size_t wkv_forward_workspace_size_path(int64_t B, int64_t T, int64_t C, int dtype, int path);

/* The wkv_path (WKV_PATH_SERIAL, _CHUNKED or _CHAINED) that wkv_forward takes
 * for these sizes on the current device, with k, v, y 4-byte aligned (for
 * reports and tests).  Negative wkv_status for invalid sizes or dtype. */
int wkv_forward_auto_path(int64_t B, int64_t T, int64_t C, int dtype);

/*
 * Training / prefill form: y for every position, and optionally the state
 * after the last token ([tm-math] "Why it collapses into a recurrence": one
 * scan over time, parallel across batch and channels; [vanos] "The WKV
 * Operator", training mode; [multigrid] "Prefill, decode, ...": prefill
 * yields the state after the last prompt token).
 *
 *   B >= 1, T >= 0, C >= 1; C * sizeof(dtype) * 33 + 512 < 2^32 (a block of
 *               up to 32 token rows is addressed with 32-bit byte offsets;
 *               larger C returns WKV_ERR_SHAPE)
 *   w, u        [C] fp32            decay rate (> 0) and bonus
 *   k, v        [B,T,C] dtype       keys, values
 *   y           [B,T,C] dtype       output; must not overlap k, v, w, u or the state
 *   a_in, b_in, p_in   [B,C] fp32   prior state; all NULL = empty history
 *   a_out, b_out, p_out [B,C] fp32  state after token T-1; all NULL = not wanted.
 *                                   May be the same arrays as *_in.
 *   workspace   device buffer of at least wkv_forward_workspace_size() bytes
 *               (may be NULL when that size is 0)
 * T = 0 writes no y and copies the prior state (or the empty state) to *_out.
 */
int wkv_forward(int64_t B, int64_t T, int64_t C, int dtype,
                const float *w, const float *u,
                const void *k, const void *v, void *y,
                const float *a_in, const float *b_in, const float *p_in,
                float *a_out, float *b_out, float *p_out,
                void *workspace, size_t workspace_bytes, void *stream);

/* wkv_forward with the execution path forced (testing and tuning).  The
 * workspace must be sized with wkv_forward_workspace_size_path() for the same
 * path. */
int wkv_forward_path(int64_t B, int64_t T, int64_t C, int dtype, int path,
                     const float *w, const float *u,
                     const void *k, const void *v, void *y,
                     const float *a_in, const float *b_in, const float *p_in,
                     float *a_out, float *b_out, float *p_out,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * wkv_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace; where the chosen path needs one (the chunked path), it
 * uses a fixed device array of WKV_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends.  Sizes whose
 * workspace (wkv_forward_workspace_size) exceeds that return WKV_ERR_WORKSPACE.
 * The call allocates nothing and frees nothing; each call clears what it uses
 * of the array with a kernel of its own.  All calls on one device share the
 * array, so calls that may overlap on one device (different streams without
 * ordering between them) race: order them on one stream.  Arguments, outputs
 * and other errors are those of wkv_forward.
 */
#define WKV_NOALLOC_SCRATCH_BYTES (40u << 20)

int wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, int dtype,
                        const float *w, const float *u,
                        const void *k, const void *v, void *y,
                        const float *a_in, const float *b_in, const float *p_in,
                        float *a_out, float *b_out, float *p_out,
                        void *stream);

/*
 * Training / prefill form with the receptance gate fused on the way out
 * ([tm-math] "Receptance: the gate on the way out"): for every position
 *
 *   o = sigmoid(r) * wkv,   sigmoid(r) = 1 / (1 + e^{-r}),  elementwise,
 *
 * where wkv is what wkv_forward writes to y.  Reading r in the same pass
 * saves writing wkv and reading it back.  The projection W_o that follows on
 * the pages is not part of the call.
 *
 *   path        a wkv_path (WKV_PATH_AUTO to let the library choose)
 *   r           [B,T,C] dtype       receptance; required when T > 0
 *   o           [B,T,C] dtype       output; must not overlap k, v, r, w, u or the state
 * All other arguments, the state outputs (the plain recurrence's state: the
 * gate does not enter it), the workspace (wkv_forward_workspace_size_path of
 * the same path) and the error behaviour are as in wkv_forward_path.
 */
int wkv_forward_gated(int64_t B, int64_t T, int64_t C, int dtype, int path,
                      const float *w, const float *u,
                      const void *k, const void *v, const void *r, void *o,
                      const float *a_in, const float *b_in, const float *p_in,
                      float *a_out, float *b_out, float *p_out,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode: one token for every (layer l, sequence s, channel c) of [L,S,C]
 * ([aiwiki] wkv_step: state in, (y, state') out; [vanos] "The WKV Operator",
 * inference mode; [multigrid] "Prefill, decode, ...").
 *
 *   L, S, C >= 1
 *   w, u        [L,C] fp32          per-layer decay rate and bonus
 *   k, v        [L,S,C] dtype
 *   y           [L,S,C] dtype       must not overlap any input
 *   a_in, b_in, p_in    [L,S,C] fp32  required (use p = -inf for an empty history)
 *   a_out, b_out, p_out [L,S,C] fp32  required; each may equal its *_in (in place),
 *                                     but must not partially overlap any array
 * The state is rounded to fp32 after every step.  Its exponent p_out is an
 * anchor, not necessarily the running maximum: it stays where it is until a
 * new key exceeds it (then p_out = k exactly) or the decayed sums fall below
 * 2^-40 (then it moves down by 28), and the decay e^{-w} is applied to
 * a_out, b_out instead.  Any (a, b, p) with the same e^p a and e^p b is the
 * same state, and every call accepts any such state.  This keeps the
 * per-token roundings from all going one way, so a chain of steps follows
 * wkv_forward's outputs to a few 1e-6 relative, also behind keys near +40.
 */
int wkv_step(int64_t L, int64_t S, int64_t C, int dtype,
             const float *w, const float *u,
             const void *k, const void *v, void *y,
             const float *a_in, const float *b_in, const float *p_in,
             float *a_out, float *b_out, float *p_out,
             void *stream);

/*
 * wkv_step with the receptance gate ([tm-math] "Receptance: the gate on the
 * way out"): y = sigmoid(r) * wkv for the one token.
 *   r           [L,S,C] dtype       receptance, required; y must not overlap it
 * Everything else as in wkv_step; the state is the plain recurrence's.
 */
int wkv_step_gated(int64_t L, int64_t S, int64_t C, int dtype,
                   const float *w, const float *u,
                   const void *k, const void *v, const void *r, void *y,
                   const float *a_in, const float *b_in, const float *p_in,
                   float *a_out, float *b_out, float *p_out,
                   void *stream);

/*
 * Token shift ([tm-math] "Token shift: a two-tap causal convolution";
 * [multigrid] "Token shift and channel mixing"): for each of the three
 * blends mu_r, mu_k, mu_v
 *
 *   xbar_t = mu * x_t + (1 - mu) * x_{t-1}
 *
 * over x [B,T,C].  x_{-1} is x_prev [B,C] when given, else 0.
 *
 *   x           [B,T,C] dtype
 *   x_prev      [B,C] dtype or NULL
 *   mu_r, mu_k, mu_v  [C] fp32
 *   xr, xk, xv  [B,T,C] dtype       must not overlap x or each other
 *   x_last      [B,C] dtype or NULL receives x_{T-1} (x_prev or 0 when T = 0)
 * Evaluated as x_{t-1} + mu * (x_t - x_{t-1}) in fp32.
 */
int wkv_token_shift(int64_t B, int64_t T, int64_t C, int dtype,
                    const void *x, const void *x_prev,
                    const float *mu_r, const float *mu_k, const float *mu_v,
                    void *xr, void *xk, void *xv, void *x_last, void *stream);

/*
 * Session state save and resume ([multigrid] "The state, in bytes" and its
 * closing note: a session's state is small and constant in length, so it can
 * be serialised, stored and resumed elsewhere at full fidelity).  The state
 * of ONE sequence `seq` of a decode batch -- a, b, p of every layer plus
 * n_shift shifted-token arrays (the previous step's token of each sub-block
 * that token-shifts) -- is copied to or from a host blob:
 *
 *   header (64 bytes: magic "WKVS", format version 1, L, C, dtype, n_shift),
 *   a, b, p [L][C] fp32 each, then n_shift arrays [L][C] in dtype.
 *
 *   L, S, C           decode-batch shape; seq in [0, S)
 *   a, b, p           [L,S,C] fp32 device arrays (the wkv_step state)
 *   shift             host array of n_shift device pointers, each [L,S,C]
 *                     in dtype (may be NULL when n_shift == 0);
 *                     0 <= n_shift <= WKV_SESSION_MAX_SHIFT
 *   blob              host memory of at least wkv_session_bytes() bytes
 *                     (pinned memory makes the copies asynchronous)
 *
 * Both calls enqueue row copies (hipMemcpy2DAsync) on `stream` and return:
 * a saved blob is complete, and a loaded state usable, once the stream
 * reaches them.  wkv_session_save writes the header at once.
 * wkv_session_load checks the header (magic, version, L, C, dtype, n_shift)
 * and the blob size first and enqueues nothing on a mismatch.  The other
 * sequences of the batch are not touched.
 */
#define WKV_SESSION_MAX_SHIFT 8
size_t wkv_session_bytes(int64_t L, int64_t C, int dtype, int n_shift);
int wkv_session_save(int64_t L, int64_t S, int64_t C, int dtype, int64_t seq,
                     const float *a, const float *b, const float *p,
                     const void *const *shift, int n_shift,
                     void *blob, size_t blob_bytes, void *stream);
int wkv_session_load(int64_t L, int64_t S, int64_t C, int dtype, int64_t seq,
                     const void *blob, size_t blob_bytes,
                     float *a, float *b, float *p, void *const *shift, int n_shift,
                     void *stream);

/*
 * Gradients of wkv_forward from the empty history (training):
 * with L = sum over b, t, c of gy * y, where y is wkv_forward's output for
 * (k, v, w, u) and no initial state, returns dL/dk, dL/dv [B,T,C] and
 * dL/dw, dL/du [C] (summed over the batch and the tokens).  Each y_t is a
 * weighted mean of the values ([tm-math] "The WKV operator"), so its partial
 * derivatives are those of a softmax-weighted mean whose exponents move one
 * for one with k_i, with u on the current token, and by -(t-1-i) with w.
 *
 *   B, C >= 1, T >= 0, C * 68 < 2^32
 *   w, u        [C] fp32
 *   k, v, gy    [B,T,C] dtype       inputs and the gradient of L wrt y
 *   gk, gv      [B,T,C] dtype       outputs (rounded to dtype)
 *   gw, gu      [C] fp32            outputs; zero when T = 0
 *   workspace   device memory of wkv_backward_workspace_size(B, T, C) bytes,
 *               256-byte aligned (NULL allowed when T = 0); it holds the
 *               forward state before every 16-token sub-chunk (2 fp32 per
 *               channel, half a byte per token-channel) and per-column partial
 *               sums, and is overwritten
 * No output may overlap any input, another output or the workspace.
 * Arithmetic is fp32 with every exponential of a non-positive argument;
 * gw, gu are reduced over the batch in a fixed order (deterministic).
 */
size_t wkv_backward_workspace_size(int64_t B, int64_t T, int64_t C);
int wkv_backward(int64_t B, int64_t T, int64_t C, int dtype,
                 const float *w, const float *u,
                 const void *k, const void *v, const void *gy,
                 void *gk, void *gv, float *gw, float *gu,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * The training pair that reads k and v once less.  wkv_backward first re-runs
 * the forward recurrence over every token to recover the state before each
 * 16-token sub-chunk; a forward that is run anyway can save those states as
 * it goes, and the backward then starts from them.  Same operator, same
 * results to rounding as wkv_forward + wkv_backward.
 *
 * wkv_forward_save: wkv_forward from the empty history (no state in or out)
 * that also writes
 *   states      [B][ceil(T/16)][2][C] fp32 device array,
 *               wkv_saved_states_bytes(B, T, C) bytes, 8-byte aligned: for
 *               sub-chunk s (tokens 16 s .. 16 s + 15) of row b the
 *               recurrence's state before its first token as two numbers
 *               per channel: r, the history's weighted mean of v (a / b),
 *               and q, the log of its total weight (p + ln b), so that the
 *               history sums are r e^q and e^q; the empty history (s = 0)
 *               is r = 0, q = -1e38.  No chunk of it may overlap an input
 *               or y.
 * It always runs the chained path (one workgroup per group of 64 or 128
 * channels of a row); k, v, y, w, u and the errors are as for wkv_forward.
 *
 * wkv_backward_saved: wkv_backward with `states` from wkv_forward_save for
 * the same (k, v, w, u, B, T, C, dtype), read and not written.  Its
 * workspace (wkv_backward_saved_workspace_size(B, C) bytes, 256-byte
 * aligned, NULL allowed when T = 0) holds only the per-column partial sums.
 * States from other inputs give gradients of nothing in particular; the
 * call cannot tell.
 */
#define WKV_SAVED_STATE_TOKENS 16
size_t wkv_saved_states_bytes(int64_t B, int64_t T, int64_t C);
int wkv_forward_save(int64_t B, int64_t T, int64_t C, int dtype,
                     const float *w, const float *u, const void *k, const void *v,
                     void *y, float *states, void *stream);
size_t wkv_backward_saved_workspace_size(int64_t B, int64_t C);
int wkv_backward_saved(int64_t B, int64_t T, int64_t C, int dtype,
                       const float *w, const float *u,
                       const void *k, const void *v, const void *gy, const float *states,
                       void *gk, void *gv, float *gw, float *gu,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Matrix-valued state WKV of RWKV-5 "Eagle" and RWKV-6 "Finch" ([vanos] the
 * table "Versions: RWKV-4 -> Eagle -> Finch" and the matrix-form recurrence
 * under it).  Channels are grouped into H heads of WKV_MAT_HEAD_DIM = 64
 * (C = 64 H; channel c is index c % 64 of head c / 64).  Per batch row and
 * head, a state S of 64 x 64 (row i: key channel, column j: value channel):
 *
 *   S_t = diag(d_t) S_{t-1} + k_t v_t^T,      y_t = r_t^T S_t,
 *   d_t = exp(-softplus(z_t)) = 1 / (1 + e^{z_t})
 *
 * z is the table's decay argument a.b + w: per token for Finch
 * (WKV_MAT_DECAY_PER_TOKEN, stored like r), per channel for Eagle
 * (WKV_MAT_DECAY_PER_CHANNEL, fp32).  The page gives no bonus term and no
 * normalisation for this form; neither is applied.  The state is fp32,
 * element (i, j) of head h of row b at ((b H + h) 64 + i) 64 + j; a NULL
 * state input is the zero state.
 */
#define WKV_MAT_HEAD_DIM 64
typedef enum {
    WKV_MAT_DECAY_PER_CHANNEL = 0,  /* z [C] fp32 (forward), [L,C] fp32 (step)   */
    WKV_MAT_DECAY_PER_TOKEN = 1     /* z shaped and stored like r                 */
} wkv_mat_decay;

typedef enum {
    WKV_MAT_PATH_AUTO = 0,          /* chunked for bf16, token by token for fp32  */
    WKV_MAT_PATH_CHUNKED = 1,       /* 16-token chunks as dense 16x16x16 products */
                                    /* on the matrix cores (bf16 operands, fp32   */
                                    /* accumulation); bf16 storage only          */
    WKV_MAT_PATH_TOKENWISE = 2      /* the recurrence token by token in fp32      */
} wkv_mat_path;

/*
 * Training / prefill form over [B,T,C], and optionally the state after the
 * last token.
 *
 *   B, H >= 1, T >= 0; H * 64 * 4 * 17 < 2^32 (rows of a chunk are addressed with
 *               32-bit byte offsets; larger H returns WKV_ERR_SHAPE)
 *   r, k, v     [B,T,C] dtype       receptance, keys, values
 *   z           see wkv_mat_decay
 *   s_in        [B,H,64,64] fp32    prior state, or NULL (zero)
 *   s_out       [B,H,64,64] fp32    state after token T-1, or NULL; may be s_in
 *   y           [B,T,C] dtype       output; must not overlap any input or s_out
 * r, k, v, z, y must be 8-byte (bf16) or 16-byte (fp32) aligned.  The chunked
 * path runs a chunk token by token instead, in fp32, when a channel decays by
 * more than e^{-80} within it, and the whole call so when 16 rows of C bf16
 * values reach 2 GiB (C >= 2^26).  Results do not depend on timing.
 */
int wkv_mat_forward(int64_t B, int64_t T, int64_t H, int dtype,
                    const void *r, const void *k, const void *v, const void *z, int z_mode,
                    const float *s_in, float *s_out, void *y, void *stream);
int wkv_mat_forward_path(int64_t B, int64_t T, int64_t H, int dtype, int path,
                         const void *r, const void *k, const void *v, const void *z, int z_mode,
                         const float *s_in, float *s_out, void *y, void *stream);

/*
 * Decode form: one token for each of L x S rows (layers x sequences), each
 * of H heads ([vanos] "O(N) Inference Characteristics": one matrix-vector
 * product against a fixed-size state per token).
 *
 *   L, S, H >= 1
 *   r, k, v     [L,S,C] dtype
 *   z           [L,S,C] dtype (per token) or [L,C] fp32 (per channel)
 *   s_in        [L,S,H,64,64] fp32  required
 *   s_out       [L,S,H,64,64] fp32  required; may be s_in (in place)
 *   y           [L,S,C] dtype
 * r, k, v, z, y must be 8-byte (bf16) or 16-byte (fp32) aligned, s_in and
 * s_out 16-byte aligned.
 */
int wkv_mat_step(int64_t L, int64_t S, int64_t H, int dtype,
                 const void *r, const void *k, const void *v, const void *z, int z_mode,
                 const float *s_in, float *s_out, void *y, void *stream);

/* Static description of a status code. */
const char *wkv_status_string(int status);

/* Message for the last failing call on this thread ("" if none). */
const char *wkv_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int wkv_abi_version(void);

/*
 * Bounded waits that gave up, on the current device, since the library was
 * loaded.  Two kernels wait on work of other waves or workgroups: the chunked
 * forward path's look-back over earlier tiles, and the matrix-state forward's
 * ring of operand slots.  Each wait is bounded (200 ms) so that a kernel
 * always ends; a wait that gives up is never expected, and when it happens the
 * results it would have fed are written as NaN (the chunked path: the tile and
 * every later tile of its column group; the ring: the head's y and s_out),
 * the chunked path also sets the uint32 error word at byte offset 4 of its
 * workspace (cleared by every call), and the count read here grows by one.
 *   count    host pointer, receives the count
 * Synchronous: copies from device memory after the device's prior work (do
 * not call during stream capture).  Returns WKV_OK or WKV_ERR_NULL/WKV_ERR_HIP.
 */
int wkv_bounded_wait_failures(uint64_t *count);

#define WKV_ABI_VERSION 107

#ifdef __cplusplus
}
#endif

#endif /* WKV_H */
